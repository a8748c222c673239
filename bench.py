#!/usr/bin/env python3
"""Throughput of the draft-tree build and target-side verify path on one GPU.

One step = one pass of the whole path over one batch with every input
resident in HBM: draft top-k -> tree build (scores, parents, positions, mask,
retrieve arrays) -> tree-verify attention -> accept walk -> KV compaction
(c5 instead: pruned LM head -> logit constraint -> distribution scatter ->
top-1 -> tree -> stochastic accept -> target-to-draft id remap).

Prints one JSON line: metric "verified draft tokens/s" (B * N tree tokens per
step, root included), a roofline entry for the step's dominant kernel (HIP
events on the launch stream) and, on rank 0 at N=1, the CPU oracle timed on
a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3]
                    [--accept literal|planted] [--no-cpu-baseline]
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

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
ROTATE = 3                     # input sets the timed steps rotate through
# read-only inputs that are rotated (outputs, tables and small arrays are not)
ROTATED = ("draft_probs", "draft_logits_in", "draft_logits", "target_logits", "target", "q", "k_pool", "v_pool", "hidden", "weight", "q_pruned",
           "mask_bits")
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published

WORKLOAD_NAMES = {
    "c1": "tiny EAGLE tree verify (B=2, topk=2, S=3, N=6, V=1000, Hq=Hkv=4, D=64, L=256, greedy)",
    "c2": "linear stochastic verify (B=16, topk=1, S=4, N=5, V=128256, T=1.0)",
    "c3": "EAGLE-2 tree verify, Llama-3-8B attention shape (B=32, topk=8, S=5, N=64, V=128256, "
          "Hq=32, Hkv=8, D=128, page 1, L~U[512,4096], greedy, slot compaction)",
    "c4": "paged tree verify (B=64, topk=4, S=4, N=32, V=128256, Hq=32, Hkv=8, D=128, page 16, "
          "L~U[1024,8192], stochastic T=0.7, page-16 compaction)",
    "c5": "TLI draft step + linear verify (B=64, H=896, K=60000, V_draft=151936, V_target=128256, "
          "topk=1, S=4, N=5, stochastic)",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c3", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--accept", default="literal", choices=["literal", "planted", "full"],
                    help="literal inputs; planted: a seeded accepted path of U{0..S} nodes per request; full: "
                         "every request accepts S nodes (a stress case for the compaction)")
    ap.add_argument("--logits", action="store_true",
                    help="stochastic workloads: read the draft and target logits and compute both processed "
                         "distributions softmax(logits / T) on the GPU inside the step (two more stages)")
    ap.add_argument("--draft-input", default="probs", choices=["probs", "logits_f32", "logits_bf16"],
                    help="what the draft top-k reads: the processed probability rows, or the draft logits "
                         "(fp32 or bf16) with the softmax fused into the top-k (non-TLI workloads)")
    ap.add_argument("--chain", action="store_true",
                    help="k = 1 workloads: build the draft as a multi-layer chain (sdv_build_chain) instead of "
                         "through the tree builder")
    ap.add_argument("--kv-alloc", action="store_true",
                    help="workloads with attention: add the draft-side KV allocation (backup, per-branch "
                         "regions with the partial-page copies, rollback) to the step")
    ap.add_argument("--extend-prep", action="store_true",
                    help="add the index preparation of the draft extend after the accept walk to the step")
    ap.add_argument("--layers", type=int, default=1,
                    help="KV layers the compaction moves (page > 1); layer 0 is the attention's pool, the others "
                         "are pools of the same shape that only the compaction touches")
    ap.add_argument("--batch", type=int, default=None, help="override the workload's batch (side figures)")
    ap.add_argument("--k-inter", type=int, default=None, help="TLI workloads: override the intersection size")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed steps before the warm-up until the GPU has run this long (ms): it lowers its "
                         "clocks when idle, and the timed steps should see the clocks of a busy serving loop")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=32, help="requests in the CPU oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB -> 1 GiB device copy kernel 5 times (scales the HBM counters)")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- GPU path

class Pipeline:
    """Preallocated device buffers and the per-stage calls of one step."""

    def __init__(self, cfg, inp, n_tables, accept_mode, draft_input="probs", extend_prep=False, chain=False,
                 kv_alloc=False, layers=1, logits=False):
        import torch
        import speculative_decoding_eagle_amd as sdv
        self.torch, self.sdv, self.cfg = torch, sdv, cfg
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).cuda()
        self.d = {k: dev(v) for k, v in inp.items() if isinstance(v, np.ndarray) and v.ndim > 0}
        self.fallback = int(inp.get("fallback", 0))
        B, N, k, S = cfg.B, cfg.N, cfg.k, cfg.S
        d = self.d
        if cfg.is_tli:
            self.q_target = torch.empty((B, cfg.R, cfg.V), dtype=torch.float32, device="cuda")
            self.logits = torch.empty((B, cfg.K_inter), dtype=torch.float32, device="cuda")
            self.full = torch.empty((B, cfg.V_draft), dtype=torch.float32, device="cuda")
            self.d2t, self.t2d = sdv.sdv_tli_build_maps(d["inter_ids"], d["tgt_ids"], cfg.V_draft, cfg.V,
                                                        self.fallback)
            self.scatter_ws = torch.empty(sdv._lib.lib().sdv_tli_q_scatter_workspace_size(cfg.V), dtype=torch.uint8,
                                          device="cuda")
            sdv.sdv_tli_q_scatter(d["q_pruned"], d["tgt_ids"], cfg.V, q_target=self.q_target, ws=self.scatter_ws)
            self.remap_out = torch.empty((B, S + 1), dtype=torch.int32, device="cuda")
            self.draft_rows = self.q_target
        else:
            self.draft_rows = d["draft_probs"]
        self.draft_input = draft_input
        self.from_logits = logits
        if logits:
            # the processed rows are this step's outputs: the stages below
            # write them from the logits
            d["draft_probs"] = torch.empty_like(d["draft_logits"])
            d["target"] = torch.empty_like(d["target_logits"])
            self.draft_rows = d["draft_probs"]
        self.extend_prep = extend_prep
        self.chain = chain
        self.kv_alloc = kv_alloc and cfg.has_attention
        if self.kv_alloc:
            # room for every branch of every request past the workload's own
            # pages; the allocator hands out exactly those pages
            P = cfg.page
            extra = B * k * sdv.sdv_kv_branch_pages(P, S)
            num_pages = d["k_pool"].shape[0] // P
            for key in ("k_pool", "v_pool"):
                old = d[key]
                grown = torch.empty(((num_pages + extra) * P,) + tuple(old.shape[1:]), dtype=old.dtype, device="cuda")
                grown[:old.shape[0]].copy_(old)
                d[key] = grown
            self.kv = sdv.sdv_kv_alloc_init(extra)
            self.kv.free_ids.copy_(torch.arange(num_pages + extra - 1, num_pages - 1, -1, dtype=torch.int32))
            self.kv_backup = torch.empty(2, dtype=torch.int32, device="cuda")
            self.kv_pages = torch.empty((B, k, sdv.sdv_kv_branch_pages(P, S)), dtype=torch.int32, device="cuda")
            self.kv_loc = torch.empty((B, k, S), dtype=torch.int32, device="cuda")
        self.ext = {}
        if draft_input != "probs":
            # the fused path reads logits; the stochastic accept still reads
            # the probability rows of the draft distribution
            lg = d.pop("draft_logits")
            self.draft_logits = lg.to(torch.bfloat16) if draft_input == "logits_bf16" else lg
            d["draft_logits_in"] = self.draft_logits
        rows = B * cfg.R
        self.topk_p = torch.empty((B, cfg.R, k), dtype=torch.float32, device="cuda")
        self.topk_id = torch.empty((B, cfg.R, k), dtype=torch.int32, device="cuda")
        ws = max(sdv._lib.lib().sdv_draft_topk_workspace_size(rows, cfg.V, k),
                 sdv._lib.lib().sdv_draft_topk_logits_workspace_size(rows, cfg.V, k))
        self.topk_ws = torch.zeros(max(ws, 1), dtype=torch.uint8, device="cuda")   # calls leave it zeroed
        self.tree = {}
        self.acc = {}
        self.acc_ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")   # calls leave it zero-filled
        self.mode = sdv.STOCHASTIC if cfg.mode == "stochastic" else sdv.GREEDY
        if cfg.has_attention:
            self.attn_out = torch.empty((B, N, cfg.Hq, cfg.D), dtype=torch.bfloat16, device="cuda")
            self.tables = [d["page_table"].clone() for _ in range(n_tables)]
            self.new_len = torch.empty(B, dtype=torch.int32, device="cuda")
            self.freed = torch.empty(B * N, dtype=torch.int32, device="cuda")
            self.num_freed = torch.empty(1, dtype=torch.int32, device="cuda")
        self.target = d["target"]
        # extra KV layers that only the compaction reads and writes
        self.extra_k, self.extra_v = [], []
        self.layers = layers if (cfg.has_attention and cfg.page > 1) else 1
        if cfg.has_attention and cfg.page > 1:
            for _ in range(layers - 1):
                self.extra_k.append(torch.empty_like(d["k_pool"]))
                self.extra_v.append(torch.empty_like(d["v_pool"]))
        # warm build, used to plant acceptance when asked
        self.run_all(0)
        torch.cuda.synchronize()
        if accept_mode in ("planted", "full"):
            self._plant(full=accept_mode == "full")
        # Input rotation: the read-only inputs of more than 1 MB get ROTATE
        # copies and step i reads copy i % ROTATE, so at least two other
        # steps' inputs (GBs at the large workloads) pass through L2 and the
        # 256 MB MALL before a step's own inputs come back: every stage
        # starts cold, as it would in a serving loop where the target and
        # draft models run in between.
        self.sets = [d]
        for _ in range(1, ROTATE):
            self.sets.append({key: (val.clone() if key in ROTATED and val.numel() * val.element_size() > (1 << 20)
                                    and not (logits and key in ("draft_probs", "target")) else val)
                              for key, val in d.items()})
        torch.cuda.synchronize()

    def use(self, i):
        """Point the stages at input set i % ROTATE."""
        self.d = self.sets[i % len(self.sets)]
        if self.from_logits:
            # the outputs of the softmax stages are shared by every set
            self.d["draft_probs"], self.d["target"] = self.sets[0]["draft_probs"], self.sets[0]["target"]
        self.target = self.d["target"]
        if not self.cfg.is_tli:
            self.draft_rows = self.d["draft_probs"]
        if self.draft_input != "probs":
            self.draft_logits = self.d["draft_logits_in"]

    def _plant(self, full=False):
        """Make the target accept a random-length path of first children
        (setup only; the same planted rows are then used by every step)."""
        cfg, torch = self.cfg, self.torch
        rng = workloads.extra_rng(cfg, 99)
        nt = self.tree["next_token"].cpu().numpy()
        tok = self.tree["tokens"].cpu().numpy()
        qr = self.tree["q_row"].cpu().numpy()
        t = self.target
        for b in range(cfg.B):
            a = cfg.S if full else int(rng.integers(0, cfg.S + 1))
            u = 0
            for _ in range(a):
                c = int(nt[b, u])
                if c < 0:
                    break
                if self.mode == self.sdv.GREEDY:
                    t[b, u, int(tok[b, c])] = t[b, u].max() + 1.0
                elif self.from_logits:
                    # equal logits at the same temperature give p = q bit for bit
                    self.d["target_logits"][b, u] = self.d["draft_logits"][b, int(qr[b, u])]
                else:
                    t[b, u] = self.draft_rows[b, int(qr[b, u])]
                u = c
        torch.cuda.synchronize()

    # ---- stages
    def s_tli(self):
        sdv, d, cfg = self.sdv, self.d, self.cfg
        sdv.sdv_tli_lm_head(d["hidden"][0], d["weight"], logits=self.logits)
        sdv.sdv_tli_constrain_draft_logits(self.logits, d["inter_ids"], cfg.V_draft, full=self.full)
        # the target -> intersection inverse was built at set-up (the maps are static)
        sdv.sdv_tli_q_scatter(d["q_pruned"], None, cfg.V, q_target=self.q_target, ws=self.scatter_ws)

    def s_softmax_draft(self):
        self.sdv.sdv_softmax_rows(self.d["draft_logits"], self.cfg.temperature, out=self.d["draft_probs"])

    def s_softmax_target(self):
        self.sdv.sdv_softmax_rows(self.d["target_logits"], self.cfg.temperature, out=self.d["target"])

    def s_topk(self):
        if self.draft_input == "probs":
            self.sdv.sdv_draft_topk(self.draft_rows, self.cfg.k, topk_p=self.topk_p, topk_id=self.topk_id,
                                    ws=self.topk_ws)
        else:
            self.sdv.sdv_draft_topk_logits(self.draft_logits, self.cfg.k, self.cfg.temperature,
                                           topk_p=self.topk_p, topk_id=self.topk_id, ws=self.topk_ws)

    def s_tree(self):
        cfg = self.cfg
        if self.chain:
            self.tree = self.sdv.sdv_build_chain(self.topk_p, self.topk_id, self.d["root_token"],
                                                 self.d["prefix_len"], out=self.tree)
            return
        self.tree = self.sdv.sdv_build_tree(self.topk_p, self.topk_id, self.d["root_token"], self.d["prefix_len"],
                                            cfg.k, cfg.S, cfg.N, out=self.tree)

    def s_attn(self, i):
        cfg = self.cfg
        self.sdv.sdv_tree_verify_attention(self.d["q"], self.d["k_pool"], self.d["v_pool"], self.tables[i],
                                           self.d["prefix_len"], self.tree["mask_bits"], page=cfg.page,
                                           out=self.attn_out)

    def s_accept(self):
        d = self.d
        kw = {}
        if self.mode == self.sdv.STOCHASTIC:
            kw = dict(draft_probs=self.draft_rows, u_accept=d["u_accept"], u_draw=d["u_draw"])
        self.acc = self.sdv.sdv_verify_accept(self.mode, self.tree, self.target, self.cfg.S, out=self.acc,
                                              ws=self.acc_ws, **kw)

    def s_compact(self, i):
        cfg, d = self.cfg, self.d
        pools = ([d["k_pool"]] + self.extra_k, [d["v_pool"]] + self.extra_v) if cfg.page > 1 else ([], [])
        self.sdv.sdv_compact_kv(self.tables[i], d["prefix_len"], self.acc["accept_len"], self.acc["accept_path"],
                                cfg.N, cfg.S, cfg.page, pools[0], pools[1], new_len=self.new_len, freed=self.freed,
                                num_freed=self.num_freed)

    def s_kv_draft(self, i):
        cfg, sdv = self.cfg, self.sdv
        pools = ([self.d["k_pool"]], [self.d["v_pool"]]) if cfg.page > 1 else ([], [])
        sdv.sdv_kv_alloc_backup(self.kv, self.kv_backup)
        sdv.sdv_kv_alloc_branches(self.kv, cfg.page, cfg.k, cfg.S, self.tables[i], self.d["prefix_len"], *pools,
                                  branch_pages=self.kv_pages, out_loc=self.kv_loc)
        sdv.sdv_kv_alloc_restore(self.kv, self.kv_backup)

    def s_extend(self):
        self.ext = self.sdv.sdv_draft_extend_prep(self.d["prefix_len"], self.acc["commit_len"],
                                                  self.acc["commit_tokens"], self.acc["accept_path"], self.cfg.N,
                                                  t2d=self.t2d if self.cfg.is_tli else None, out=self.ext)

    def s_remap(self):
        self.sdv.sdv_tli_map_ids(self.t2d, self.acc["commit_tokens"], out=self.remap_out)

    def stages(self, i):
        cfg = self.cfg
        st = []
        if self.kv_alloc:
            st.append(("kv_alloc_draft", lambda: self.s_kv_draft(i)))
        if cfg.is_tli:
            st.append(("tli_head_mask_scatter", self.s_tli))
        if self.from_logits:
            st.append(("softmax_draft", self.s_softmax_draft))
        st += [("draft_topk", self.s_topk), ("build_tree", self.s_tree)]
        if cfg.has_attention:
            st.append(("tree_attention", lambda: self.s_attn(i)))
        if self.from_logits:
            st.append(("softmax_target", self.s_softmax_target))
        st.append(("accept", self.s_accept))
        if cfg.has_attention:
            st.append(("compact_kv", lambda: self.s_compact(i)))
        if cfg.is_tli:
            st.append(("t2d_remap", self.s_remap))
        if self.extend_prep:
            st.append(("extend_prep", self.s_extend))
        return st

    def settle_step(self, n):
        """Untimed step n on the input set of a timed step n (rotating as they
        do): every stage but the two that rewrite the page table (the
        compaction and the draft-side allocation), so table 0 is only read.
        (Settle steps that also compacted, on a table restored before each
        step, were followed by stalls of some 30 ms in later steps of the
        page-16 and planted workloads; without those stages there were none.)"""
        self.use(n)
        for name, fn in self.stages(0):
            if name not in ("compact_kv", "kv_alloc_draft"):
                fn()

    def run_all(self, i):
        if hasattr(self, "sets"):
            self.use(i)
        for _, fn in self.stages(i):
            fn()


def algorithmic_work(cfg, inp, pipe):
    """Bytes / flops the method must move or compute per launch, per stage."""
    B, N, V, R, k = cfg.B, cfg.N, cfg.V, cfg.R, cfg.k
    row_bytes = 2 if pipe.draft_input == "logits_bf16" else 4
    out = {"draft_topk": dict(bytes=B * R * V * row_bytes + B * R * k * 8, flops=0)}
    if pipe.from_logits:
        # every row read once and written once
        out["softmax_draft"] = dict(bytes=B * R * V * 8, flops=0)
        out["softmax_target"] = dict(bytes=B * N * V * 8, flops=0)
    if cfg.has_attention:
        L = inp["prefix_len"].astype(np.int64)
        depth = pipe.tree["depth"].cpu().numpy().astype(np.int64)
        W = (N + 31) // 32
        kv = int(((L + N) * cfg.Hkv * cfg.D * 2 * 2).sum())
        qo = B * N * cfg.Hq * cfg.D * 2 * 2
        idx = int(((L + N) * 4).sum()) + B * N * W * 4 + B * 4
        vis = (L[:, None] + depth + 1).sum()
        out["tree_attention"] = dict(bytes=kv + qo + idx, flops=int(vis) * cfg.Hq * cfg.D * 4)
    acc_len = pipe.acc["accept_len"].cpu().numpy().astype(np.int64)
    commit = pipe.acc["commit_len"].cpu().numpy().astype(np.int64)
    rows = int(np.maximum(commit, 1).sum())     # visited nodes = committed tokens
    per_row = V * 4 * (2 if cfg.mode == "stochastic" else 1)
    out["accept"] = dict(bytes=rows * per_row, flops=0, accepted=int(acc_len.sum()))
    if cfg.has_attention:
        # page > 1: K and V rows [Hkv, D] of every moved token, read and
        # written, every layer; page 1: the slot-map entries of the tree
        path = pipe.acc["accept_path"].cpu().numpy()
        moved = int(sum(int((path[b, 1:acc_len[b] + 1] != np.arange(1, acc_len[b] + 1)).sum()) for b in range(B)))
        if cfg.page > 1:
            out["compact_kv"] = dict(bytes=moved * 2 * 2 * cfg.Hkv * cfg.D * 2 * pipe.layers, flops=0, moved=moved)
        else:
            out["compact_kv"] = dict(bytes=B * N * 4 * 2 + B * 4 * 3, flops=0, moved=moved)
    if cfg.is_tli:
        H = cfg.H_draft
        out["tli_head_mask_scatter"] = dict(
            bytes=cfg.K_inter * H * 2 + B * H * 2 + B * cfg.K_inter * 4          # GEMM
            + B * cfg.K_inter * 4 + B * cfg.V_draft * 4 + cfg.K_inter * 4       # constrain
            + B * R * cfg.K_inter * 4 + B * R * V * 4 + cfg.K_inter * 4,        # scatter
            flops=2 * B * H * cfg.K_inter)
    return out


# HBM traffic of the dominant kernel, from two rocprofv3 --pmc passes
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) over this bench's default
# workload, each scaled by what the same counter reads for the plain copy of
# --copy-calibration.  The figure belongs to the kernel source it was taken on
# (its sha256); once that file changes the bench reports null until the
# counters are taken again.
MEASURED_TRAFFIC = {
    "tree_attention": {
        "workload": "c3",
        "sources": ["speculative_decoding_eagle_amd/csrc/attn_wide.hip",
                    "speculative_decoding_eagle_amd/csrc/attn_common.hpp",
                    "speculative_decoding_eagle_amd/csrc/common.hpp"],
        "sha256": "bea906d6037b1b958f236de89197049b8d36b811ddc744a1d44e4e7a3e519fcd",
        "fetch_kib": 198137.7, "fetch_factor": 1.99996,
        "write_kib": 34438.6, "write_factor": 1.0,
    },
}


def sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(stage, workload):
    rec = MEASURED_TRAFFIC.get(stage)
    if rec is None or rec["workload"] != workload or rec["sha256"] is None:
        return None
    if sources_sha256(rec["sources"]) != rec["sha256"]:
        return None
    return int(rec["fetch_kib"] * 1024 * rec["fetch_factor"] + rec["write_kib"] * 1024 * rec["write_factor"])


# --------------------------------------------------------------- CPU oracle

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, n_req, threads=1, logits=False):
    """The oracle, as it stands, on the first n_req requests of the same
    workload, BLAS limited to `threads` threads (the tree build and walks are
    single-threaded Python); scaled to verified tokens/s.  With `logits`, the
    step starts from the draft and target logits as the GPU step does."""
    from threadpoolctl import threadpool_limits
    import oracle.accept as oacc
    import oracle.attention as oatt
    import oracle.compact as ocmp
    import oracle.softmax as osm
    import oracle.tli as otli
    import oracle.topk as otopk
    import oracle.tree as otree
    n = min(n_req, cfg.B)
    sl = slice(0, n)
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        if cfg.is_tli:
            h = inp["hidden"][0][sl]
            head_logits = otli.lm_head(h, inp["weight"])
            otli.constrain_logits(head_logits.astype(np.float32), inp["inter_ids"], cfg.V_draft)
            rows = otli.q_scatter(inp["q_pruned"][sl].reshape(-1, cfg.K_inter), inp["tgt_ids"], cfg.V)
            rows = rows.reshape(n, cfg.R, cfg.V)
        elif logits:
            rows = osm.softmax_rows(inp["draft_logits"][sl], cfg.temperature).astype(np.float32)
        else:
            rows = inp["draft_probs"][sl]
        tp, ti = otopk.draft_topk(rows, cfg.k)
        tree = otree.build_tree(tp, ti, inp["root_token"][sl], inp["prefix_len"][sl], cfg.k, cfg.S, cfg.N)
        if cfg.has_attention:
            oatt.tree_verify_attention(inp["q"][sl], inp["k_pool"], inp["v_pool"], inp["page_table"][sl],
                                       inp["prefix_len"][sl], tree["mask"], page=cfg.page)
        if cfg.mode == "greedy":
            acc = oacc.verify_greedy(tree, inp["target"][sl], cfg.S)
        else:
            target = osm.softmax_rows(inp["target_logits"][sl], cfg.temperature).astype(np.float32) if logits \
                else inp["target"][sl]
            acc = oacc.verify_stochastic(tree, target, rows, inp["u_accept"][sl], inp["u_draw"][sl], cfg.S)
        if cfg.has_attention:
            ocmp.compact_kv(inp["page_table"][sl], [], [], inp["prefix_len"][sl], acc["accept_len"],
                            acc["accept_path"], cfg.N, cfg.page) if cfg.page == 1 else \
                ocmp.compact_kv(inp["page_table"][sl], [inp["k_pool"]], [inp["v_pool"]], inp["prefix_len"][sl],
                                acc["accept_len"], acc["accept_path"], cfg.N, cfg.page)
        dt = time.perf_counter() - t0
    return {"value": n * cfg.N / dt, "unit": "verified draft tokens/s", "cores": threads, "kind": "oracle",
            "sample": "first %d of %d requests of %s, every stage of the step (oracle, numpy, BLAS on %d "
                      "thread%s), %.2f s" % (n, cfg.B, cfg.name, threads, "" if threads == 1 else "s", dt),
            "cpu_model": cpu_model()}


# ------------------------------------------------------ counter calibration

COPY_BYTES = 1 << 30


def copy_calibration():
    """A plain streaming kernel of known traffic: 5 launches of dst = -src over
    1 GiB of float32 (1 GiB read + 1 GiB written per launch).  The FETCH_SIZE
    and WRITE_SIZE counters of these launches give the factor that turns the
    counters into bytes."""
    import torch
    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"read_bytes": COPY_BYTES, "write_bytes": COPY_BYTES, "launches": 5}}))


# --------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the path is measured at one GPU's share and no "
              "multi-GPU path is built. Got --gpus %d." % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    over = {}
    if args.batch is not None:
        over["B"] = args.batch
    if args.k_inter is not None:
        over["K_inter"] = args.k_inter
    cfg = workloads.get_config(args.config, **over)
    log("generating inputs of %s" % cfg.name)
    t_gen = time.perf_counter()
    if args.draft_input != "probs" and cfg.is_tli:
        print("--draft-input %s: the TLI workloads take the draft rows from the pruned head" % args.draft_input,
              file=sys.stderr)
        sys.exit(2)
    if args.logits and (cfg.mode != "stochastic" or cfg.is_tli or args.draft_input != "probs"):
        print("--logits: the non-TLI stochastic workloads (c2, c4) with --draft-input probs", file=sys.stderr)
        sys.exit(2)
    inp = workloads.generate(cfg, with_logits=args.draft_input != "probs" or args.logits)
    t_gen = time.perf_counter() - t_gen
    log("inputs ready in %.1f s; uploading and warming up" % t_gen)
    if args.chain and (cfg.k != 1 or cfg.N != cfg.S + 1):
        print("--chain needs a k = 1 workload whose tree keeps every step (N = S + 1)", file=sys.stderr)
        sys.exit(2)
    pipe = Pipeline(cfg, inp, args.warmup + args.steps + 1, args.accept, args.draft_input, args.extend_prep,
                    args.chain, args.kv_alloc, args.layers, args.logits)
    stages = [name for name, _ in pipe.stages(0)]

    # The GPU lowers its clocks when idle (it has been, during input
    # generation) and raises them only under uninterrupted load: measured at
    # c3, 20 timed steps after 5 warm-up steps take 0.27 ms each, after 50
    # 0.250 and after 200 0.243, while hundreds of untimed steps in bursts of
    # ten with a host sync between them leave it at 0.27.  So, untimed, one
    # continuous burst of about settle_ms of steps (their count from the time
    # of ten).
    settle_steps, t_settle = 0, time.perf_counter()
    if args.settle_ms > 0:
        for _ in range(10):
            pipe.settle_step(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
        per = (time.perf_counter() - t_settle) / 10
        for _ in range(int(args.settle_ms * 1e-3 / max(per, 1e-5))):
            pipe.settle_step(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    t_settle = time.perf_counter() - t_settle

    for i in range(args.warmup):
        pipe.run_all(1 + i)
    torch.cuda.synchronize()
    base = 1 + args.warmup

    # whole-step throughput (no events inside the timed region)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        pipe.run_all(base + i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # per-stage times with HIP events on the launch stream (same work again)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        pipe.use(base + i)
        st = pipe.stages(base + i)
        ev[i][0].record()
        for j, (_, fn) in enumerate(st):
            fn()
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
                for j, name in enumerate(stages)}

    log("timed %d steps: %.3f ms/step" % (args.steps, ms_step))
    work = algorithmic_work(cfg, inp, pipe)
    dom = max((s for s in stages if s in work), key=lambda s: stage_ms[s])
    w = work[dom]
    t_s = stage_ms[dom] * 1e-3
    gbs = w["bytes"] / t_s / 1e9
    roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dom, cfg.name), "kernel": dom,
                "algorithmic_bytes": int(w["bytes"]), "avg_ms": round(stage_ms[dom], 4)}
    if w.get("flops"):
        roofline["mfma_tflops"] = round(w["flops"] / t_s / 1e12, 2)
        roofline["mfma_frac"] = round(w["flops"] / t_s / 1e12 / BF16_PEAK_TFLOPS, 4)

    tokens = cfg.B * cfg.N
    value = tokens / (ms_step * 1e-3)
    # the headline workload's metric as stated with it; its HBM rate is the
    # roofline entry's "achieved"
    METRIC_C3 = "verified draft tokens/sec (build+tree-attn+accept) at B=32 topk=8; HBM GB/s"
    line = {
        "metric": METRIC_C3 if cfg.name == "c3" else "verified draft tokens/sec (build+tree-attn+accept)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"steps": settle_steps, "ms": round(t_settle * 1e3, 1)},
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32+bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[cfg.name], "name": cfg.name, "batch": cfg.B, "tree_tokens": cfg.N,
                   "accept": args.accept, "draft_input": args.draft_input, "logits": args.logits,
                   "extend_prep": args.extend_prep, "chain": args.chain,
                   "kv_alloc": args.kv_alloc, "kv_layers": args.layers},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stage_gbs": {k: round(work[k]["bytes"] / (stage_ms[k] * 1e-3) / 1e9, 1) for k in stages if k in work},
        "accepted_tokens": work["accept"]["accepted"],
        "roofline": roofline,
        "device": torch.cuda.get_device_name(0),
        "input_generation_s": round(t_gen, 2),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample (one core, then every core of this process)")
        line["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample, threads=1, logits=args.logits)
        ncores = len(os.sched_getaffinity(0))
        if ncores > 1:
            allc = cpu_baseline(cfg, inp, args.cpu_sample, threads=ncores, logits=args.logits)
            line["cpu_baseline"]["all_cores"] = {k: allc[k] for k in ("value", "cores", "sample")}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

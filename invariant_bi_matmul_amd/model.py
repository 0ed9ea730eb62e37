"""A dense Llama-style decoder stack run on libbi's batch-invariant kernels.

Every arithmetic step is a libbi call:
- token embedding and row gathers: ``bi_embed``;
- ``bi_rmsnorm``, then ``bi_matmul_packed`` (weights in the strip layout of
  ``bi_matmul_pack_w``; bitwise ``bi_matmul``) for the q/k/v, output,
  gate/up/down and lm_head projections (q|k|v and gate|up as one matmul each
  by default);
- ``bi_qkv_rope`` (split of the fused q|k|v output plus rotary embedding), or
  ``bi_rope``;
- ``bi_attn_prefill`` / ``bi_attn_decode`` over a paged KV cache (16-token
  pages, fixed 256-position splits, fixed-order combine);
- ``bi_add`` (residual), ``bi_swiglu_pair`` / ``bi_swiglu``, and ``bi_argmax``
  (greedy sampling).

This module keeps only bookkeeping: the weights, the KV pages each sequence
owns, and the per-call index arrays (token ids, positions, cu_q, kv_len,
block tables).  Since every kernel is batch-invariant, a sequence gets the
same logits and tokens, bit for bit, whether it runs alone or among any
other sequences, and however its prompt is chunked.  That is the end-to-end
property the tests and ``bench.py`` check.

The layer is the usual pre-norm one:
  h = x + W_o attn(rope(W_q n1(x)), rope(W_k n1(x)), W_v n1(x))
  y = h + W_down (silu(W_gate n2(h)) * W_up n2(h))
with n1, n2 RMSNorm, GQA attention (n_q query heads over n_kv key/value
heads) and softmax scale 1/sqrt(head_dim).  Then logits = W_lm n_f(x_last)
in fp32 and the next token is their argmax (lowest index on ties).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import (PAGE, add, argmax, attn_decode, attn_decode_i16, attn_prefill, attn_prefill_i16,
               attn_workspace_bytes, bix_attn_decode_splitkv, bix_matmul_splitk,
               bix_rmsnorm_splitrow, embed, make_shape, matmul, matmul_ec, matmul_ec_pack_w,
               matmul_pack_w, matmul_packed,
               qkv_rope, rmsnorm, rope, swiglu, swiglu_pair)

__all__ = ["LlamaConfig", "LAYER_WEIGHTS", "weight_shapes", "Decoder", "DecodeGraph"]


@dataclass(frozen=True)
class LlamaConfig:
    """Llama-3-8B shape by default.  The pages name no vocabulary size or
    rotary base; these are Llama 3's, and neither affects invariance."""
    hidden: int = 4096
    layers: int = 32
    n_q: int = 32
    n_kv: int = 8
    head_dim: int = 128
    ffn: int = 14336
    vocab: int = 128256
    rope_theta: float = 500000.0
    eps: float = 1e-5


LAYER_WEIGHTS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


def weight_shapes(cfg: LlamaConfig) -> Tuple[Dict[str, tuple], Dict[str, tuple]]:
    """(shapes of the global weights, shapes of one layer's weights); every
    projection is stored [in, out], the layout ``bi_matmul`` reads."""
    H, F, V = cfg.hidden, cfg.ffn, cfg.vocab
    qd, kvd = cfg.n_q * cfg.head_dim, cfg.n_kv * cfg.head_dim
    glob = {"embed": (V, H), "final_norm": (H,), "lm_head": (H, V)}
    layer = {"attn_norm": (H,), "wq": (H, qd), "wk": (H, kvd), "wv": (H, kvd), "wo": (qd, H),
             "mlp_norm": (H,), "w_gate": (H, F), "w_up": (H, F), "w_down": (F, H)}
    return glob, layer


@dataclass
class _Seq:
    length: int = 0
    pages: List[int] = field(default_factory=list)


PROJECTIONS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


class Decoder:
    """Holds the weights and a paged KV cache for up to ``max_tokens`` cached
    positions in total; sequences are added, stepped and released by id.

    ``comparator=True`` swaps in the library's non-invariant comparators
    (split-row RMSNorm, split-K matmul and split-KV decode attention, whose
    split counts follow the batch size), as a negative control: with them a
    sequence's bits depend on its companions.

    ``fuse=True`` runs the q, k and v projections as one matmul against
    [W_q | W_k | W_v] (then ``bi_qkv_rope`` splits and rotates), and gate and
    up as one against [W_gate | W_up] (then ``bi_swiglu_pair``): one launch
    fills the GPU where three small ones each left most of it idle.  Every
    output column is the same dot product in the same k order either way, so
    the bits are those of the separate projections.

    ``kv="int16"`` keeps the KV cache as int16 codes with a factor per
    (token, kv head) (``bi_attn_prefill_i16`` / ``bi_attn_decode_i16``).

    ``mm="ec"`` takes the projection weights (and lm_head) in fp32 and runs
    every projection as an error-compensated matmul (``bi_matmul_ec``) against
    the weight packed once as [hi; lo; hi]: the product of the bf16 activation
    with the fp32 weight, to about 2^-16 of sum |a||w|.  The activations stay
    bf16 (so lo(a) = 0 and each call takes two products)."""

    def __init__(self, cfg: LlamaConfig, weights: dict, max_tokens: int,
                 device: Optional[torch.device] = None, comparator: bool = False,
                 fuse: bool = True, kv: str = "bf16", mm: str = "bf16"):
        if kv not in ("bf16", "int16") or mm not in ("bf16", "ec"):
            raise ValueError("kv must be 'bf16' or 'int16', mm 'bf16' or 'ec'")
        if comparator and (kv != "bf16" or mm != "bf16"):
            raise ValueError("the comparators exist for the bf16 cache and matmul only")
        glob, layer = weight_shapes(cfg)
        wdt = torch.float32 if mm == "ec" else torch.bfloat16

        def check(name, t, shape):
            want = wdt if name in PROJECTIONS or name == "lm_head" else torch.bfloat16
            if tuple(t.shape) != shape or t.dtype != want:
                raise ValueError("weight %s must be %s %s" % (name, want, shape))

        for name, shape in glob.items():
            check(name, weights[name], shape)
        if len(weights["layers"]) != cfg.layers:
            raise ValueError("need %d layers of weights" % cfg.layers)
        for lw in weights["layers"]:
            for name, shape in layer.items():
                check(name, lw[name], shape)
        self.cfg = cfg
        self.w = weights
        self.device = device or weights["embed"].device
        self.fuse = fuse
        self.kv, self.mm = kv, mm
        # the tensors each projection multiplies by: the bf16 weight, or the
        # packed [hi; lo; hi] of the fp32 one; q|k|v and gate|up concatenated
        # once when fused
        # bf16: each weight whose width is a multiple of 32 goes into the strip
        # layout (matmul_pack_w), which a small-batch step streams in whole
        # bursts; the products are bitwise those of the row-major weight
        if mm == "ec":
            prep = matmul_ec_pack_w
        else:
            def prep(t):
                return matmul_pack_w(t) if t.shape[1] % 32 == 0 else t
        self.proj = []
        for lw in weights["layers"]:
            pw = {"wo": prep(lw["wo"]), "w_down": prep(lw["w_down"])}
            if fuse:
                pw["w_qkv"] = prep(torch.cat([lw["wq"], lw["wk"], lw["wv"]], dim=1).contiguous())
                pw["w_gu"] = prep(torch.cat([lw["w_gate"], lw["w_up"]], dim=1).contiguous())
            else:
                for name in ("wq", "wk", "wv", "w_gate", "w_up"):
                    pw[name] = prep(lw[name])
            self.proj.append(pw)
        self.lm_head = prep(weights["lm_head"])
        self.num_pages = (max_tokens + PAGE - 1) // PAGE + 1
        cache = (self.num_pages, cfg.n_kv, PAGE, cfg.head_dim)
        cdt = torch.int16 if kv == "int16" else torch.bfloat16
        self.kc = [torch.zeros(cache, dtype=cdt, device=self.device) for _ in range(cfg.layers)]
        self.vc = [torch.zeros(cache, dtype=cdt, device=self.device) for _ in range(cfg.layers)]
        if kv == "int16":
            self.ks = [torch.zeros(cache[:3], dtype=torch.float32, device=self.device)
                       for _ in range(cfg.layers)]
            self.vs = [torch.zeros(cache[:3], dtype=torch.float32, device=self.device)
                       for _ in range(cfg.layers)]
        self.free = list(range(self.num_pages - 1, -1, -1))
        self.seqs: Dict[int, _Seq] = {}
        self.scale = float(torch.tensor(1.0 / math.sqrt(cfg.head_dim), dtype=torch.float32))
        self.comparator = comparator
        if comparator:
            self._norm = lambda x, g: bix_rmsnorm_splitrow(x, g, cfg.eps)
            self._mm = lambda a, w, **kw: bix_matmul_splitk(a, w, **kw)  # either layout
        elif mm == "ec":
            self._norm = lambda x, g: rmsnorm(x, g, cfg.eps)
            self._mm = lambda a, w3, out_dtype=torch.bfloat16: matmul_ec(a, w3,
                                                                         out_dtype=out_dtype)
        else:
            self._norm = lambda x, g: rmsnorm(x, g, cfg.eps)
            self._mm = lambda a, w, **kw: (matmul_packed(a, w, **kw) if w.dim() == 3
                                           else matmul(a, w, **kw))

    # ---- KV page bookkeeping ---------------------------------------------------
    def add_sequence(self, sid: int):
        if sid in self.seqs:
            raise ValueError("sequence %d exists" % sid)
        self.seqs[sid] = _Seq()

    def release(self, sid: int):
        s = self.seqs.pop(sid)
        self.free.extend(reversed(s.pages))

    def length(self, sid: int) -> int:
        return self.seqs[sid].length

    def _reserve(self, s: _Seq, new_len: int):
        need = (new_len + PAGE - 1) // PAGE
        while len(s.pages) < need:
            if not self.free:
                raise RuntimeError("KV pool exhausted")
            s.pages.append(self.free.pop())

    # ---- one forward call ------------------------------------------------------
    def forward(self, batch: Sequence[Tuple[int, Sequence[int]]]):
        """Feed new tokens to sequences: ``batch`` lists (sequence id, new token
        ids).  Returns (logits fp32 [B, vocab] at each sequence's last new
        token, next tokens int32 [B] = their argmax).  A call in which every
        sequence brings one token is a decode step (``bi_attn_decode``);
        otherwise a (chunked) prefill (``bi_attn_prefill``)."""
        cfg, dev = self.cfg, self.device
        if not batch:
            raise ValueError("empty batch")
        seqs = [self.seqs[sid] for sid, _ in batch]
        n_new = [len(ids) for _, ids in batch]
        if min(n_new) < 1:
            raise ValueError("every sequence needs at least one new token")
        starts = [s.length for s in seqs]
        after = [a + n for a, n in zip(starts, n_new)]
        for s, L in zip(seqs, after):
            self._reserve(s, L)
        B, T = len(batch), sum(n_new)
        maxp = max(len(s.pages) for s in seqs)
        table = [s.pages + [s.pages[-1]] * (maxp - len(s.pages)) for s in seqs]
        cu = [0]
        for n in n_new:
            cu.append(cu[-1] + n)
        i32 = dict(dtype=torch.int32, device=dev)
        ids = torch.tensor([t for _, toks in batch for t in toks], **i32)
        pos = torch.tensor([p for a, n in zip(starts, n_new) for p in range(a, a + n)], **i32)
        cu_q = torch.tensor(cu, **i32)
        kv_len = torch.tensor(after, **i32)
        bt = torch.tensor(table, **i32)
        last = torch.tensor([c - 1 for c in cu[1:]], **i32)
        decode = max(n_new) == 1
        ws = self._decode_workspace(B, maxp, max(after)) if decode else None
        logits, nxt = self._body(ids, pos, cu_q, kv_len, bt, last, max(n_new), max(after), ws)
        for s, L in zip(seqs, after):
            s.length = L
        return logits, nxt

    def _decode_workspace(self, B: int, maxp: int, max_len: int):
        if self.comparator:
            return None
        cfg = self.cfg
        shape = make_shape(B, cfg.n_q, cfg.n_kv, cfg.head_dim, maxp, self.num_pages, self.scale)
        need = attn_workspace_bytes(shape, B, max_len)
        return torch.empty(max(need, 16) // 4 + 4, dtype=torch.float32, device=self.device)

    def _attend(self, li, q, k, v, cu_q, kv_len, bt, max_new, max_len, ws, decode):
        """Append k/v to layer li's cache, then attention for q."""
        kc, vc = self.kc[li], self.vc[li]
        if self.kv == "int16":
            ks, vs = self.ks[li], self.vs[li]
            if decode:
                return attn_decode_i16(q, k, v, kv_len, bt, kc, vc, ks, vs, self.scale, max_len,
                                       workspace=ws)
            return attn_prefill_i16(q, k, v, cu_q, kv_len, bt, kc, vc, ks, vs, self.scale,
                                    max_new)
        if decode and self.comparator:
            return bix_attn_decode_splitkv(q, k, v, kv_len, bt, kc, vc, self.scale, max_len)
        if decode:
            return attn_decode(q, k, v, kv_len, bt, kc, vc, self.scale, max_len, workspace=ws)
        return attn_prefill(q, k, v, cu_q, kv_len, bt, kc, vc, self.scale, max_new)

    def _body(self, ids, pos, cu_q, kv_len, bt, last, max_new: int, max_len: int, ws):
        """The stack on device tensors: T = len(ids) tokens of B = len(kv_len)
        sequences; a decode step when max_new == 1.  Only device work, so a
        decode step can be captured into a graph and replayed."""
        cfg = self.cfg
        T = ids.shape[0]
        decode = max_new == 1
        nq, nkv, d = cfg.n_q, cfg.n_kv, cfg.head_dim
        norm, mm = self._norm, self._mm

        x = embed(ids, self.w["embed"])
        for li, lw in enumerate(self.w["layers"]):
            pw = self.proj[li]
            h = norm(x, lw["attn_norm"])
            if self.fuse:
                q, k, v = qkv_rope(mm(h, pw["w_qkv"]), pos, nq, nkv, cfg.rope_theta)
            else:
                q = mm(h, pw["wq"]).view(T, nq, d)
                k = mm(h, pw["wk"]).view(T, nkv, d)
                v = mm(h, pw["wv"]).view(T, nkv, d)
                rope(q, k, pos, cfg.rope_theta)
            o = self._attend(li, q, k, v, cu_q, kv_len, bt, max_new, max_len, ws, decode)
            add(x, mm(o.view(T, nq * d), pw["wo"]), out=x)
            h = norm(x, lw["mlp_norm"])
            if self.fuse:
                g = swiglu_pair(mm(h, pw["w_gu"]))
            else:
                g = mm(h, pw["w_gate"])
                swiglu(g, mm(h, pw["w_up"]), out=g)
            add(x, mm(g, pw["w_down"]), out=x)
        xl = embed(last, x)  # the last new token of each sequence (a row gather)
        logits = mm(norm(xl, self.w["final_norm"]), self.lm_head, out_dtype=torch.float32)
        return logits, argmax(logits)

    # ---- the cache on the host (suspend and resume) ----------------------------
    def export_state(self, sids: Sequence[int]) -> dict:
        """Copy the named sequences' cached keys and values (every layer, their
        pages only, in position order) and their lengths to host memory."""
        out = {"lengths": {}, "layers": []}
        for sid in sids:
            out["lengths"][sid] = self.seqs[sid].length
        for li in range(self.cfg.layers):
            per = {}
            for sid in sids:
                pg = torch.tensor(self.seqs[sid].pages, dtype=torch.long, device=self.device)
                arrs = [self.kc[li], self.vc[li]]
                if self.kv == "int16":
                    arrs += [self.ks[li], self.vs[li]]
                per[sid] = [a.index_select(0, pg).cpu() for a in arrs]
            out["layers"].append(per)
        return out

    def import_state(self, state: dict):
        """Re-create sequences from ``export_state``'s copy: each gets fresh
        pages from the pool (wherever they fall) holding the same keys and
        values at the same positions."""
        for sid, L in state["lengths"].items():
            self.add_sequence(sid)
            s = self.seqs[sid]
            self._reserve(s, L)
            s.length = L
        for li, per in enumerate(state["layers"]):
            arrs = [self.kc[li], self.vc[li]]
            if self.kv == "int16":
                arrs += [self.ks[li], self.vs[li]]
            for sid, saved in per.items():
                pg = torch.tensor(self.seqs[sid].pages, dtype=torch.long, device=self.device)
                for a, host in zip(arrs, saved):
                    a.index_copy_(0, pg, host.to(self.device))

    def decode_graph(self, sids: Sequence[int], max_len: int) -> "DecodeGraph":
        """Decode steps of the sequences ``sids`` (in this order) until any
        reaches ``max_len`` positions, replayed from one captured graph."""
        return DecodeGraph(self, list(sids), max_len)

    # ---- greedy generation -----------------------------------------------------
    def generate(self, prompts: Dict[int, Sequence[int]], steps: int,
                 chunk: Optional[int] = None, keep_logits: Sequence[int] = (),
                 graph: bool = True):
        """Prefill every prompt (in one call, or in calls of ``chunk`` tokens per
        sequence), then ``steps`` greedy decode steps over all of them (with
        ``graph``, replayed from a captured graph: the same kernels on the
        same inputs, so the same bits).
        Returns ({id: generated tokens}, {id: [fp32 logits per generated token]})
        where logits are kept (on the device) only for ids in ``keep_logits``."""
        for sid in prompts:
            self.add_sequence(sid)
        sids = list(prompts)
        toks: Dict[int, List[int]] = {sid: [] for sid in sids}
        kept: Dict[int, List[torch.Tensor]] = {sid: [] for sid in keep_logits}
        off = {sid: 0 for sid in sids}
        while True:
            part = []
            for sid in sids:
                p = prompts[sid]
                if off[sid] < len(p):
                    n = len(p) - off[sid] if chunk is None else min(chunk, len(p) - off[sid])
                    part.append((sid, list(p[off[sid]:off[sid] + n])))
            if not part:
                break
            logits, nxt = self.forward(part)
            nxt = nxt.tolist()
            for i, (sid, ids) in enumerate(part):
                off[sid] += len(ids)
                if off[sid] == len(prompts[sid]):  # the prompt's last token: first output
                    toks[sid].append(nxt[i])
                    if sid in kept:
                        kept[sid].append(logits[i].clone())
        dg = None
        if graph and steps > 2:
            dg = self.decode_graph(sids, max(self.seqs[sid].length for sid in sids) + steps)
        for _ in range(steps - 1):
            if dg is not None:
                logits, nxt = dg.step([toks[sid][-1] for sid in sids])
            else:
                logits, nxt = self.forward([(sid, [toks[sid][-1]]) for sid in sids])
            nxt = nxt.tolist()
            for i, sid in enumerate(sids):
                toks[sid].append(nxt[i])
                if sid in kept:
                    kept[sid].append(logits[i].clone())
        for sid in sids:
            self.release(sid)
        return toks, kept


class DecodeGraph:
    """One decode step of a fixed list of sequences, captured into a HIP graph
    on first use and replayed for every later step.  A step of the stack is
    about a dozen launches per layer; replayed, they leave the host at once.

    The step's index arrays (token ids, positions, kv_len, block table) live
    in static device buffers that each step overwrites before the replay.
    The attention launch is sized for ``max_len`` positions; its kernels read
    the actual lengths from kv_len, so a step's arithmetic is that of an
    eager ``Decoder.forward`` on the same inputs.  Outputs (logits, next
    tokens) are static tensors, valid until the next step."""

    def __init__(self, dec: Decoder, sids: List[int], max_len: int):
        self.dec, self.sids = dec, sids
        B = len(sids)
        self.maxp = (max_len + PAGE - 1) // PAGE
        self.max_len = self.maxp * PAGE
        i32 = dict(dtype=torch.int32, device=dec.device)
        self.ids = torch.zeros(B, **i32)
        self.pos = torch.zeros(B, **i32)
        self.kv_len = torch.ones(B, **i32)
        self.bt = torch.zeros(B, self.maxp, **i32)
        self.cu = torch.arange(B + 1, **i32)
        self.last = torch.arange(B, **i32)
        self.ws = dec._decode_workspace(B, self.maxp, self.max_len)
        self.graph = None
        self.out = None

    def _run(self):
        return self.dec._body(self.ids, self.pos, self.cu, self.kv_len, self.bt, self.last, 1,
                              self.max_len, self.ws)

    def step(self, tokens: Sequence[int]):
        dec, B = self.dec, len(self.sids)
        seqs = [dec.seqs[sid] for sid in self.sids]
        if len(tokens) != B:
            raise ValueError("one token per sequence")
        for s in seqs:
            if s.length + 1 > self.max_len:
                raise RuntimeError("sequence longer than the captured step allows")
            dec._reserve(s, s.length + 1)
        rows = [s.pages + [s.pages[-1]] * (self.maxp - len(s.pages)) for s in seqs]
        flat = (list(tokens) + [s.length for s in seqs] + [s.length + 1 for s in seqs]
                + [p for r in rows for p in r])
        dev = torch.tensor(flat, dtype=torch.int32, device=dec.device)  # one host-to-device copy
        self.ids.copy_(dev[:B])
        self.pos.copy_(dev[B:2 * B])
        self.kv_len.copy_(dev[2 * B:3 * B])
        self.bt.copy_(dev[3 * B:].view(B, self.maxp))
        if self.graph is None:
            # warm up once outside the capture (the step's K/V append is
            # idempotent: the replay writes the same values to the same slots)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                self._run()
            torch.cuda.current_stream().wait_stream(side)
            self.graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(self.graph):
                self.out = self._run()
        self.graph.replay()
        for s in seqs:
            s.length += 1
        return self.out

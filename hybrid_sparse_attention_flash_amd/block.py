"""Sequencing of the C-ABI calls into hybrid blocks (host logic only).

HySparse block (QbitAI HySparse article, method section): the full layer runs
causal attention and emits block scores; one top-k per query picks the blocks;
every sparse layer attends over those blocks of the shared KV and over its own
128-token window, merged by the sigmoid gate (one fused call per layer, or the
sparse and window+gate calls separately).

HySparse2 block (airebao HySparse2 news, inner KV Reuse / token-level selection /
forced recent window): the full layer emits per-tile token scores; one top-k
per 64-query tile picks tokens; every sparse layer attends over them united
with the recent window, over the one shared KV.

All buffers are allocated once per runner so repeated steps launch kernels
only.
"""
from dataclasses import dataclass
from typing import List, Optional

import torch

from . import ops


class HySparseBlock:
    """One HySparse hybrid block: 1 full layer + N gated sparse layers.

    selection: "all_heads" (one index set per query from the max over all
    query heads) or "kv_group" (one index set per query and KV group from the
    max over that group's heads; the ablation variant of the head reduction)."""

    def __init__(self, B, L, Hq, Hkv, D, n_sparse, topk, window=128, block=64, device="cuda",
                 out_dtype=torch.float32, softmax_scale=None, fused=True, selection="all_heads"):
        if selection not in ("all_heads", "kv_group"):
            raise ValueError(f"unknown selection {selection!r}")
        self.B, self.L, self.Hq, self.Hkv, self.D = B, L, Hq, Hkv, D
        self.n_sparse, self.topk, self.window, self.block = n_sparse, topk, window, block
        self.scale = softmax_scale
        self.fused = fused
        self.selection = selection
        nblk = (L + block - 1) // block
        ng = Hkv if selection == "kv_group" else 1
        f32 = dict(dtype=torch.float32, device=device)
        self.o_full = torch.empty(B, L, Hq, D, dtype=out_dtype, device=device)
        self.lse = torch.empty(B, Hq, L, **f32)
        self.scores = torch.empty(ng, B, L, nblk, **f32)
        self.idx = torch.empty(ng, B, L, topk, dtype=torch.int32, device=device)
        self.count = torch.empty(ng * B * L, dtype=torch.int32, device=device)
        # the two-call form's intermediate sparse branch
        self.o_sp = None if fused else torch.empty(B, L, Hq, D, **f32)
        self.lse_sp = None if fused else torch.empty(B, Hq, L, **f32)
        self.o_layers = [torch.empty(B, L, Hq, D, dtype=out_dtype, device=device) for _ in range(n_sparse)]

    def full(self, q0, k, v):
        mode = "block_group" if self.selection == "kv_group" else "block"
        ops.hys_full_attn_fwd(q0, k, v, self.o_full, self.lse, mode, self.scores, softmax_scale=self.scale)

    def select(self):
        rows = self.scores.shape[0] * self.B * self.L
        ops.hys_select_topk(self.scores.view(rows, -1), self.topk, self.idx.view(rows, self.topk), self.count)

    def _idx(self):
        # per-group index sets as [Hkv, B, L, k]; one set as [B, L, k]
        return self.idx if self.selection == "kv_group" else self.idx[0]

    def sparse_layer(self, l, q, k, v, kw, vw, gate_w):
        if self.fused:
            ops.hys_sparse_layer_fwd(q, k, v, self._idx(), kw, vw, self.window, gate_w, self.o_layers[l],
                                     topk=self.topk, softmax_scale=self.scale)
            return
        ops.hys_sparse_attn_fwd(q, k, v, self._idx(), self.o_sp, self.lse_sp, granularity=self.block,
                                topk=self.topk, q_tile=1, softmax_scale=self.scale)
        ops.hys_swa_gate_fwd(q, kw, vw, self.window, self.o_sp, self.lse_sp, gate_w, self.o_layers[l],
                             softmax_scale=self.scale)

    def run(self, q_layers, k, v, kw_layers, vw_layers, gate_layers):
        self.full(q_layers[0], k, v)
        self.select()
        for l in range(self.n_sparse):
            self.sparse_layer(l, q_layers[l + 1], k, v, kw_layers[l], vw_layers[l], gate_layers[l])
        return self


class HySparseTrainer:
    """Forward and backward of one HySparse block for training.

    The forward keeps what the backward needs: the full layer's O and LSE,
    the selection, and per sparse layer the two branches' O (fp32) and LSE
    (the sparse branch from hys_sparse_attn_fwd, the window branch from
    hys_window_attn_fwd), then merges them with hys_swa_gate_fwd.  The
    backward runs the full layer's gradient first (it writes dK, dV of the
    shared cache) and every sparse layer's after it (each adds its sparse
    branch's share), so dk, dv hold the block's total gradient."""

    def __init__(self, B, L, Hq, Hkv, D, n_sparse, topk, window=128, device="cuda", softmax_scale=None,
                 selection="all_heads"):
        self.fwd = HySparseBlock(B, L, Hq, Hkv, D, n_sparse, topk, window, device=device, out_dtype=torch.bfloat16,
                                 softmax_scale=softmax_scale, fused=True, selection=selection)
        self.scale = softmax_scale
        self.window = window
        f32 = dict(dtype=torch.float32, device=device)
        self.o_sp = [torch.empty(B, L, Hq, D, **f32) for _ in range(n_sparse)]
        self.lse_sp = [torch.empty(B, Hq, L, **f32) for _ in range(n_sparse)]
        self.o_w = [torch.empty(B, L, Hq, D, **f32) for _ in range(n_sparse)]
        self.lse_w = [torch.empty(B, Hq, L, **f32) for _ in range(n_sparse)]
        self.dq = [torch.empty(B, L, Hq, D, **f32) for _ in range(n_sparse + 1)]
        self.dk = torch.empty(B, L, Hkv, D, **f32)
        self.dv = torch.empty(B, L, Hkv, D, **f32)
        self.dkw = [torch.empty(B, L, Hkv, D, **f32) for _ in range(n_sparse)]
        self.dvw = [torch.empty(B, L, Hkv, D, **f32) for _ in range(n_sparse)]
        self.dgate_w = [torch.empty(Hq, D, **f32) for _ in range(n_sparse)]

    def forward(self, q_layers, k, v, kw_layers, vw_layers, gate_layers):
        f = self.fwd
        f.full(q_layers[0], k, v)
        f.select()
        for l in range(f.n_sparse):
            q = q_layers[l + 1]
            ops.hys_sparse_attn_fwd(q, k, v, f._idx(), self.o_sp[l], self.lse_sp[l], granularity=64, topk=f.topk,
                                    softmax_scale=self.scale)
            ops.hys_window_attn_fwd(q, kw_layers[l], vw_layers[l], self.window, self.o_w[l], self.lse_w[l],
                                    softmax_scale=self.scale)
            ops.hys_swa_gate_fwd(q, kw_layers[l], vw_layers[l], self.window, self.o_sp[l], self.lse_sp[l],
                                 gate_layers[l], f.o_layers[l], softmax_scale=self.scale)
        return self

    def backward(self, q_layers, k, v, kw_layers, vw_layers, gate_layers, do_full, do_layers):
        f = self.fwd
        ops.hys_full_attn_bwd(q_layers[0], k, v, f.o_full, f.lse, do_full, self.dq[0], self.dk, self.dv,
                              accumulate_kv=False, softmax_scale=self.scale)
        for l in range(f.n_sparse):
            ops.hys_sparse_layer_bwd(q_layers[l + 1], k, v, f._idx(), kw_layers[l], vw_layers[l], self.window,
                                     gate_layers[l], self.o_sp[l], self.lse_sp[l], self.o_w[l], self.lse_w[l],
                                     do_layers[l], self.dq[l + 1], self.dk, self.dv, self.dkw[l], self.dvw[l],
                                     self.dgate_w[l], accumulate_kv=True, topk=f.topk, softmax_scale=self.scale)
        return self


class HySparse2Block:
    """One HySparse2 hybrid block (prefill): 1 full layer + N token-sparse layers.

    Ablation switches (the comparisons of the HySparse2 pages):
      window_mode "forced" (the recent window joins the selected set) or
        "gated" (a sliding-window branch over the same cache fused by the
        sigmoid gate, as in HySparse; needs gate weights per layer);
      selection "token" (top-k tokens per 64-query tile) or "block" (the top
        k/64 blocks of the same scores, expanded to tokens: equal budget)."""

    def __init__(self, B, L, Hq, Hkv, D, n_sparse, topk=1024, window=128, tile=64, device="cuda",
                 out_dtype=torch.float32, softmax_scale=None, window_mode="forced", selection="token"):
        if window_mode not in ("forced", "gated") or selection not in ("token", "block"):
            raise ValueError(f"unknown window_mode {window_mode!r} or selection {selection!r}")
        if selection == "block" and topk % 64 != 0:
            raise ValueError("block selection needs a budget that is a multiple of 64 tokens")
        self.B, self.L, self.Hq, self.Hkv, self.D = B, L, Hq, Hkv, D
        self.n_sparse, self.topk, self.window, self.tile = n_sparse, topk, window, tile
        self.scale = softmax_scale
        self.window_mode, self.selection = window_mode, selection
        ntile = (L + tile - 1) // tile
        f32 = dict(dtype=torch.float32, device=device)
        self.o_full = torch.empty(B, L, Hq, D, dtype=out_dtype, device=device)
        self.lse = torch.empty(B, Hq, L, **f32)
        self.scores = torch.empty(B, ntile, L, **f32)
        self.idx = torch.empty(B, ntile, topk, dtype=torch.int32, device=device)
        self.count = torch.empty(B * ntile, dtype=torch.int32, device=device)
        self.lse_sp = torch.empty(B, Hq, L, **f32)
        self.o_sp = torch.empty(B, L, Hq, D, **f32) if window_mode == "gated" else None
        self.o_layers = [torch.empty(B, L, Hq, D, dtype=out_dtype, device=device) for _ in range(n_sparse)]

    def full(self, q0, k, v, k_scale=1.0, v_scale=1.0):
        ops.hys_full_attn_fwd(q0, k, v, self.o_full, self.lse, "tile_token", self.scores,
                              softmax_scale=self.scale, k_scale=k_scale, v_scale=v_scale)

    def select(self):
        B, nt = self.B, self.scores.shape[1]
        if self.selection == "block":
            ops.hys_select_topk_blocks(self.scores.view(B * nt, -1), self.topk // 64, self.idx.view(B * nt, self.topk))
        else:
            ops.hys_select_topk(self.scores.view(B * nt, -1), self.topk, self.idx.view(B * nt, self.topk), self.count)

    def sparse_layer(self, l, q, k, v, k_scale=1.0, v_scale=1.0, gate_w=None):
        if self.window_mode == "forced":
            ops.hys_sparse_attn_fwd(q, k, v, self.idx, self.o_layers[l], self.lse_sp, granularity=1, topk=self.topk,
                                    q_tile=self.tile, forced_window=self.window, softmax_scale=self.scale,
                                    k_scale=k_scale, v_scale=v_scale)
            return
        if gate_w is None:
            raise ValueError("the gated window needs gate weights")
        ops.hys_sparse_attn_fwd(q, k, v, self.idx, self.o_sp, self.lse_sp, granularity=1, topk=self.topk,
                                q_tile=self.tile, forced_window=0, softmax_scale=self.scale,
                                k_scale=k_scale, v_scale=v_scale)
        ops.hys_swa_gate_fwd(q, k, v, self.window, self.o_sp, self.lse_sp, gate_w, self.o_layers[l],
                             softmax_scale=self.scale, k_scale=k_scale, v_scale=v_scale)

    def run(self, q_layers, k, v, k_scale=1.0, v_scale=1.0, gate_layers=None):
        self.full(q_layers[0], k, v, k_scale, v_scale)
        self.select()
        for l in range(self.n_sparse):
            self.sparse_layer(l, q_layers[l + 1], k, v, k_scale, v_scale,
                              gate_layers[l] if gate_layers is not None else None)
        return self


class HySparse2Decode:
    """One HySparse2 decode step (full layer + top-k + N sparse layers) over an fp8 cache."""

    def __init__(self, B, Nmax, Hq, D, n_sparse, topk=1024, window=128, device="cuda", out_dtype=torch.float32,
                 softmax_scale=None):
        self.B, self.Nmax, self.Hq, self.D = B, Nmax, Hq, D
        self.n_sparse, self.topk, self.window = n_sparse, topk, window
        self.scale = softmax_scale
        self.o_full = torch.empty(B, 1, Hq, D, dtype=out_dtype, device=device)
        self.scores = torch.empty(B, Nmax, dtype=torch.float32, device=device)
        self.idx = torch.empty(B, topk, dtype=torch.int32, device=device)
        self.o_layers = [torch.empty(B, 1, Hq, D, dtype=out_dtype, device=device) for _ in range(n_sparse)]
        self.ws = None
        self._call = None          # (key, marshalled arguments) of the last call

    def run(self, q_full, k_cache, v_cache, cache_len, q_sparse, k_scale=1.0, v_scale=1.0):
        # the arguments are marshalled again only when an input tensor, a
        # length, a scale or the current stream changed since the last call
        key = (tuple((t.data_ptr(), tuple(t.shape), tuple(t.stride()), t.dtype) for t in (q_full, k_cache, v_cache)),
               tuple(int(x) for x in cache_len),
               tuple((t.data_ptr(), tuple(t.shape), tuple(t.stride()), t.dtype) for t in q_sparse),
               float(k_scale), float(v_scale), torch.cuda.current_stream(q_full.device).cuda_stream)
        if self._call is None or self._call[0] != key:
            args, self.ws, keep = ops.hys_decode_step_args(q_full, k_cache, v_cache, cache_len, self.o_full,
                                                           self.scores, self.idx, q_sparse, self.o_layers, self.topk,
                                                           self.window, softmax_scale=self.scale, k_scale=k_scale,
                                                           v_scale=v_scale, workspace=self.ws)
            self._call = (key, args, keep)
        ops.check(ops._lib.load().hys_decode_step(*self._call[1]))
        return self

"""One optimizer update of LoRA adapter slots, sequenced through liblora.

Order of one update of a slot ("4.3. Training Guide", "Gradient
accumulation"; "8. LoRA Fundamentals", "The training loop"):

  for each accumulation chunk g:
      forward of every adapted linear, layers 0..L-1
      backward of every adapted linear, layers L-1..0 (gradients summed
      into the slot's arena; chunk 0 overwrites, later chunks add)
  prepare: global norm in double, non-finite veto, one combined scale
  AdamW over the arena (A decayed, B at lr*ratio, DoRA magnitude)
  DoRA: refresh the detached row norms with the updated A, B

Each slot ("Multi-LoRA Training Example (fully-async)", "Design") owns its
arena, moments, update counter and dropout seed; slots share only W.

Memory layout of a slot: one float32 arena per role (params, grads, Adam m,
Adam v), each laid out as [all A | all B | all DoRA magnitudes] in the
linears' (layer, projection) order, so AdamW sees three segments.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

from . import lora as L
from .workloads import LoraConfig

__all__ = ["FrozenModel", "Slot", "Trainer"]


def _w_desc(W):
    """lora_dtype code and device address of a frozen weight (a float32 or
    bfloat16 tensor, or a QWeight)."""
    if isinstance(W, L.QWeight):
        return W.code, W.buf.data_ptr()
    return (L.BF16 if W.dtype == torch.bfloat16 else L.F32), W.data_ptr()


class FrozenModel:
    """The frozen weights of every adapted linear, keyed (layer, proj ordinal):
    float32 or bfloat16 tensors, or block-quantized QWeights."""

    def __init__(self, cfg: LoraConfig, weights: dict):
        self.cfg = cfg
        self.W = weights
        self.keys = sorted(weights)
        self.shape = {}
        for key in self.keys:
            N, K = weights[key].shape
            self.shape[key] = (int(K), int(N))


class Slot:
    """Trainable state of one adapter slot (params, grads, moments, counters)."""

    def __init__(self, cfg: LoraConfig, model: FrozenModel, A: dict, B: dict, seed: int,
                 device="cuda"):
        self.cfg = cfg
        self.seed = int(seed)
        self.keys = model.keys
        r = cfg.rank
        sizes_a = [r * model.shape[k][0] for k in self.keys]
        sizes_b = [model.shape[k][1] * r for k in self.keys]
        sizes_m = [model.shape[k][1] for k in self.keys] if cfg.dora else []
        na, nb, nm = sum(sizes_a), sum(sizes_b), sum(sizes_m)
        self.n = na + nb + nm
        self.segments = [(0, na, L.KIND_A), (na, nb, L.KIND_B)]
        if cfg.dora:
            self.segments.append((na + nb, nm, L.KIND_MAG))
        f32 = dict(device=device, dtype=torch.float32)
        self.params = torch.zeros(self.n, **f32)
        self.grads = torch.zeros(self.n, **f32)
        self.m = torch.zeros(self.n, **f32)
        self.v = torch.zeros(self.n, **f32)
        self.A, self.B, self.mag, self.gA, self.gB, self.gmag = {}, {}, {}, {}, {}, {}
        oa, ob, om = 0, na, na + nb
        for i, key in enumerate(self.keys):
            K, N = model.shape[key]
            self.A[key] = self.params[oa:oa + r * K].view(r, K)
            self.gA[key] = self.grads[oa:oa + r * K].view(r, K)
            self.B[key] = self.params[ob:ob + N * r].view(N, r)
            self.gB[key] = self.grads[ob:ob + N * r].view(N, r)
            self.A[key].copy_(A[key])
            self.B[key].copy_(B[key])
            oa += r * K
            ob += N * r
            if cfg.dora:
                self.mag[key] = self.params[om:om + N]
                self.gmag[key] = self.grads[om:om + N]
                om += N
        self.norm = {}
        self.t = 0   # applied updates
        self.k = 0   # 0-based index of the next update (schedule, dropout step)


@dataclass
class StepStats:
    norm: float
    vetoed: bool
    lr: float


class Trainer:
    """Runs optimizer updates of slots over one frozen model.

    The layers' linears are independent within a step (each has its own
    activations and gradients; only a layer's own chunks accumulate into the
    same gradients), so their calls can be spread over `streams` HIP streams:
    layer groups are dealt round robin, each stream with its own workspace,
    and every group keeps its chunk order on its stream.  The results are
    bitwise those of one stream.  The optimizer update runs on the current
    stream after all of them.  Short chunks leave most of the chip idle
    between a layer's dependent launches, and other layers' launches fill it.
    The default, four, is the number of hardware queues HIP gives a process
    by default; more streams share them."""

    def __init__(self, cfg: LoraConfig, model: FrozenModel, tokens=None, device="cuda", slots=1,
                 streams=4):
        self.cfg = cfg
        self.model = model
        self.T = cfg.tokens if tokens is None else int(tokens)
        # Slots over one W run their frozen products stacked (one pass over W
        # per product) when the library can: bf16 or quantized W and whole
        # 256-row tiles.
        self.nslots = int(slots)
        self.stack_slots = (self.nslots > 1 and cfg.w_dtype != "f32" and self.T % 256 == 0)
        self.scale = L.lora_scaling(cfg.alpha, cfg.rank, cfg.scaling == "rslora")
        self.device = device
        f32 = dict(device=device, dtype=torch.float32)
        r = cfg.rank
        # Projections of one layer that read the same X run as one group.
        xg = {p.ordinal: p.x_group for p in cfg.projections}
        self.groups = []
        for key in model.keys:
            g = self.groups[-1] if self.groups else None
            if g and g[0][0] == key[0] and xg[g[0][1]] == xg[key[1]] and len(g) < L.MAX_GROUP:
                g.append(key)
            else:
                self.groups.append([key])
        ws = 0
        for g in self.groups:
            ws = max(ws, L.lora_group_workspace_bytes([self._linear(k, None, dora=cfg.dora)
                                                       for k in g]))
        if cfg.dora:   # the row-norm refresh shares the workspaces between steps
            for k in model.keys:
                ws = max(ws, L.lora_dora_row_norms_workspace_bytes(self._linear(k, None)))
            nref = self.nslots if self.stack_slots else 1
            ws = max(ws, L.lora_dora_row_norms_batch_workspace_bytes(
                [self._linear(k, None) for k in model.keys for _ in range(nref)]))
        if self.stack_slots:
            for k in model.keys:
                ws = max(ws, L.lora_slots_workspace_bytes(
                    [self._linear(k, None, dora=cfg.dora)] * self.nslots))
        # Activations per slot (slot 0's are also U, Y, dX).  DoRA keeps no Z:
        # its linears take the forward's Y in the backward (dora_from_y).
        self.acts = []
        for _ in range(self.nslots if self.stack_slots else 1):
            a = {"U": {}, "Y": {}, "dX": {}}
            for key in model.keys:
                K, N = model.shape[key]
                a["U"][key] = torch.empty(self.T, r, **f32)
                a["Y"][key] = torch.empty(self.T, N, **f32)
                a["dX"][key] = torch.empty(self.T, K, **f32)
            self.acts.append(a)
        self.U, self.Y, self.dX = (self.acts[0][n] for n in ("U", "Y", "dX"))
        self.ws = torch.empty(max(ws, 256), device=device, dtype=torch.uint8)
        # Streams beyond the current one (default priority), each with a
        # workspace; no more streams than units to spread (layer groups; layers
        # on the stacked-slot path).
        units = len({k[0] for k in model.keys}) if self.stack_slots else len(self.groups)
        nstreams = max(1, min(int(streams), units))
        self.side = [torch.cuda.Stream(device=device) for _ in range(nstreams - 1)]
        self.side_ws = [torch.empty(max(ws, 256), device=device, dtype=torch.uint8)
                        for _ in self.side]
        self._calls = {}   # (id(slot), group index) -> (slot, stream handle, norms, GroupCall)
        self._refresh = {}  # (streams, slot ids) -> (slots, [(stream, linears, norms)])
        self.d_scale = torch.zeros(1, **f32)
        self.d_stats = torch.zeros(2, device=device, dtype=torch.float64)
        self.prep_ws = None

    # ------------------------------------------------------------------
    def _linear(self, key, slot, dora=False, norms_only=False):
        W = self.model.W[key]
        K, N = self.model.shape[key]
        r = self.cfg.rank
        if slot is None:   # shape-only descriptor for workspace sizing (never launched)
            aligned = 256
            wd, wp = _w_desc(W)
            return L.LoraLinear(self.T, K, N, r, wd, float(self.scale), wp, aligned, aligned,
                                aligned if dora else None, aligned if dora else None)
        mag = slot.mag.get(key) if dora else None
        nrm = slot.norm.get(key) if dora else None
        return L.make_linear(W, slot.A[key], slot.B[key], self.scale, self.T, mag, nrm,
                             dora_from_y=dora)

    def init_dora(self, slot: Slot):
        """Magnitude = ||W_i|| rows, then the detached norms of W + s B A."""
        for key in self.model.keys:
            W = self.model.W[key]
            K, N = self.model.shape[key]
            wd, wp = _w_desc(W)
            bare = L.LoraLinear(self.T, K, N, 0, wd, float(self.scale), wp, None, None, None, None)
            L.lora_dora_row_norms(bare, slot.mag[key], self.ws)
            slot.norm[key] = torch.empty(N, device=self.device, dtype=torch.float32)
        self.refresh_dora([slot])

    def refresh_dora(self, slots: list):
        """Row norms of W + s B A for every linear of `slots`, as batched
        calls: the layers are dealt to the streams in contiguous runs, one
        call per stream, and within a call the slots of each W are adjacent,
        so that one pass over W serves all of them.  Each linear writes only
        its own norm vector; the descriptors are built once per slot set
        (the tensors are updated in place)."""
        nst = 1 + len(self.side)
        key_ = (nst,) + tuple(id(sl) for sl in slots)
        hit = self._refresh.get(key_)
        if hit is None or any(a is not b for a, b in zip(hit[0], slots)):
            layers = sorted({k[0] for k in self.model.keys})
            per = -(-len(layers) // nst)
            calls = []
            for q in range(nst):
                run = set(layers[q * per:(q + 1) * per])
                lins, outs = [], []
                for key in self.model.keys:
                    if key[0] in run:
                        for sl in slots:
                            lins.append(L.make_linear(self.model.W[key], sl.A[key], sl.B[key],
                                                      self.scale, self.T))
                            outs.append(sl.norm[key])
                if lins:
                    calls.append((q, lins, outs))
            hit = (list(slots), calls)
            self._refresh[key_] = hit
        streams, wss = self._fork()
        for q, lins, outs in hit[1]:
            L.lora_dora_row_norms_batch(lins, outs, wss[q], stream=streams[q])
        self._join()

    # ------------------------------------------------------------------
    def _fork(self):
        """Streams and workspaces for the calls; the extra streams first wait
        for the work already on the current stream."""
        main = torch.cuda.current_stream()
        if self.side:
            ev = torch.cuda.Event()
            ev.record(main)
            for s in self.side:
                s.wait_event(ev)
        return [main] + self.side, [self.ws] + self.side_ws

    def _join(self):
        main = torch.cuda.current_stream()
        for s in self.side:
            ev = torch.cuda.Event()
            ev.record(s)
            main.wait_event(ev)

    def _group_call(self, slot: Slot, gi: int, stream, ws) -> L.GroupCall:
        """The marshalled call of group gi for this slot on this stream
        (built on first use: descriptors, outputs and gradients stay put)."""
        handle = stream.cuda_stream
        keys = self.groups[gi]
        # DoRA descriptors point at the slot's norm vectors, which init_dora
        # creates; the entry holds them, so they are compared by identity.
        norms = tuple(slot.norm.get(k) for k in keys) if self.cfg.dora else ()
        ent = self._calls.get((id(slot), gi))
        if (ent is None or ent[0] is not slot or ent[1] != handle or len(ent[2]) != len(norms)
                or any(a is not b for a, b in zip(ent[2], norms))):
            cfg = self.cfg
            call = L.GroupCall([self._linear(k, slot, dora=cfg.dora) for k in keys],
                               [self.Y[k] for k in keys], [self.U[k] for k in keys],
                               None,   # DoRA: the backward reads Y (dora_from_y)
                               [self.dX[k] for k in keys], [slot.gA[k] for k in keys],
                               [slot.gB[k] for k in keys],
                               [slot.gmag[k] for k in keys] if cfg.dora else None, ws, stream)
            ent = (slot, handle, norms, call)
            self._calls[(id(slot), gi)] = ent
        return ent[3]

    def forward_backward(self, slot: Slot, chunks: list):
        """Every chunk: forward over the layers 0..L-1, then backward L-1..0;
        the projections of a layer that share X go through the group calls."""
        cfg = self.cfg
        p = float(cfg.dropout)
        streams, wss = self._fork()
        ng = len(self.groups)
        calls = [self._group_call(slot, gi, streams[gi % len(streams)], wss[gi % len(streams)])
                 for gi in range(ng)]
        for g, chunk in enumerate(chunks):
            dr = [None] * ng
            if p > 0:
                dr = [calls[gi].dropouts([L.make_dropout(slot.seed, slot.k, g, k[0], k[1], p)
                                          for k in keys])
                      for gi, keys in enumerate(self.groups)]
            for gi, keys in enumerate(self.groups):
                calls[gi].forward(chunk[keys[0]][0], dr[gi])
            for gi in reversed(range(ng)):
                keys = self.groups[gi]
                calls[gi].backward(chunk[keys[0]][0], [chunk[k][1] for k in keys],
                                   accumulate=g > 0, drops=dr[gi])
        self._join()

    def forward_backward_slots(self, slots: list, chunks_per_slot: list):
        """forward_backward of several slots together: each linear's forward
        and backward go through the slot calls, whose frozen products run
        once over all slots' stacked rows."""
        cfg = self.cfg
        p = float(cfg.dropout)
        n = len(slots)
        acts = self.acts[:n]
        G = len(chunks_per_slot[0])
        streams, wss = self._fork()
        layers = sorted({k[0] for k in self.model.keys})
        ns = len(streams)
        on = {k: layers.index(k[0]) % ns for k in self.model.keys}
        # Each stream takes its linears in model order, started at a point
        # q/ns of the way through its list: with every stream on the same
        # shapes at the same time, the four run their frozen products
        # together and their rank-side kernels together; offset, one
        # stream's products overlap another's memory-bound kernels.  Every
        # linear has its own inputs, so the order changes no result.
        lists = []
        for q in range(ns):
            mine = [k for k in self.model.keys if on[k] == q]
            r = (q * len(mine)) // ns
            lists.append(mine[r:] + mine[:r])
        # issued round robin over the streams, so that each gets work early
        order = [ls[i] for i in range(max(map(len, lists))) for ls in lists if i < len(ls)]
        for g in range(G):
            def drops(key):
                if p <= 0:
                    return None
                return [L.make_dropout(sl.seed, sl.k, g, key[0], key[1], p) for sl in slots]
            for key in order:
                lins = [self._linear(key, sl, dora=cfg.dora) for sl in slots]
                L.lora_forward_slots(lins, [c[g][key][0] for c in chunks_per_slot],
                                     [a["Y"][key] for a in acts], [a["U"][key] for a in acts],
                                     None, drops(key), wss[on[key]], streams[on[key]])
            for key in reversed(order):
                lins = [self._linear(key, sl, dora=cfg.dora) for sl in slots]
                L.lora_backward_slots(lins, [c[g][key][0] for c in chunks_per_slot],
                                      [c[g][key][1] for c in chunks_per_slot],
                                      [a["U"][key] for a in acts],
                                      [a["Y"][key] for a in acts] if cfg.dora else None,
                                      [a["dX"][key] for a in acts], [sl.gA[key] for sl in slots],
                                      [sl.gB[key] for sl in slots],
                                      [sl.gmag[key] for sl in slots] if cfg.dora else None,
                                      accumulate=g > 0, drops=drops(key), ws=wss[on[key]],
                                      stream=streams[on[key]])
        self._join()

    def step_slots(self, slots: list, chunks_per_slot: list) -> list:
        """One update of every slot; with stacked slots their forward and
        backward passes share each frozen product, then each slot takes its
        own prepare, AdamW step and DoRA refresh."""
        if not self.stack_slots or len(slots) < 2:
            return [self.step(sl, ch) for sl, ch in zip(slots, chunks_per_slot)]
        if len(slots) > self.nslots:
            raise ValueError(f"trainer holds activations for {self.nslots} slots")
        self.forward_backward_slots(slots, chunks_per_slot)
        stats = [self._update(sl, len(ch), refresh=False) for sl, ch in zip(slots, chunks_per_slot)]
        if self.cfg.dora:   # one refresh for all slots (a vetoed slot's norms stay the same)
            self.refresh_dora(slots)
        return stats

    def step(self, slot: Slot, chunks: list) -> StepStats:
        self.forward_backward(slot, chunks)
        return self._update(slot, len(chunks))

    def _update(self, slot: Slot, n_chunks: int, refresh: bool = True) -> StepStats:
        """Prepare, AdamW and (unless `refresh` is False) DoRA refresh of one slot.  The prepare waits
        for its veto flag on the host (one synchronisation per update): the
        slot's update count t (bias corrections) and update index k (schedule
        and dropout step key) live on the host and must not advance on a
        vetoed update ("4.3. Training Guide", "Gradient clipping")."""
        cfg = self.cfg
        if self.prep_ws is None or self.prep_ws.numel() < L.lora_grad_prepare_workspace_bytes(slot.n):
            self.prep_ws = torch.empty(L.lora_grad_prepare_workspace_bytes(slot.n),
                                       device=self.device, dtype=torch.uint8)
        n_pred = self.T * n_chunks
        lr = L.lora_lr_at(slot.k, cfg.lr, 1 if cfg.schedule == "cosine" else 0, cfg.warmup,
                          cfg.total_updates, cfg.lr_min)
        try:
            norm = L.lora_grad_prepare(slot.grads, n_pred, cfg.max_norm, self.d_scale,
                                       self.d_stats, sync=True, ws=self.prep_ws)
        except L.LoraError as e:
            if e.status == L.LORA_E_NONFINITE:
                return StepStats(float("nan"), True, lr)
            raise
        hp = L.LoraAdamwHparams(lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay,
                                cfg.plus_ratio, slot.t + 1)
        L.lora_adamw_step(slot.params, slot.grads, slot.m, slot.v, slot.segments, hp, self.d_scale)
        if cfg.dora and refresh:
            self.refresh_dora([slot])
        slot.t += 1
        slot.k += 1
        return StepStats(norm, False, lr)

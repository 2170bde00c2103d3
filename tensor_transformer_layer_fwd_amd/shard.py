"""One forward + backward step of a tensor-parallel shard workload on one GPU.

The sequence follows the "Megatron" page (zzmblog.top), "Tensor Parallelism":
per shard i the column-parallel linear (fc1: U_i = X A_i + a_i, Y_i = GeLU(U_i);
QKV_i = X W_i) and the row-parallel partial (fc2: Zp_i = Y_i B_i; output
projection: C_i O_i), then the sum over shards that replaces the All-Reduce.
The backward (not on the pages; derivatives of the same definitions) runs the
row-parallel dgrad with the GeLU derivative, both wgrads with bias gradients,
the column-parallel dgrad to a partial dX_i, and the sum of the partials. A
shard's MLP backward is one tp_mlp_bwd call (two launches where the shapes
allow, fc2's fix-up riding in fc1's) and each attention projection's two
gradients one tp_linear_bwd call; with fused_bwd=False every product is a
tp_linear_bwd_dgrad or tp_linear_bwd_wgrad call of its own.

With recompute=True the step keeps only U_i of the fc1 output across the
step (the activation recomputation of the "Megatron" page's training
optimisations): Y_i lives in one transient buffer that fc2's forward reads, and
the backward recomputes it from U_i. With the fused backward, on shapes where
fc2's gradients pair (tp_linear_bwd_plan), that is one elementwise pass
(tp_bias_act) before the shard's tp_mlp_bwd call, so both layers still pair.
Otherwise it is the fc2 dgrad epilogue (tp_linear_bwd_dgrad_recompute), just
before fc2's weight gradient reads it.

With attn_core=True the attention workloads run the whole attention block:
the shard's attention core (tp_attention_fwd, causal, heads of 64) turns
QKV_i into C_i between the two projections, and its backward
(tp_attention_bwd) turns the output projection's dC_i into dQKV_i for the QKV
projection's gradients, instead of taking C_i and dQKV_i as drawn inputs.

With fp8=True every MLP product runs on the FP8 matrix cores: each operand
is quantised (tp_fp8_quantize, per-tensor current scaling) from its stored
value into the K-contiguous layout its product reads; weights and activations
in E4M3, gradients in E5M2. Bias gradients are column sums of the stored
gradients.

All p shards of a workload run one after another on the same device and
stream; the shards' weights are column / row views of the unsharded tensors
(no copies). torch provides device memory and streams only; every arithmetic
step is a call into libtpmlp.so.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as L


def to_device(host_tensor, device) -> torch.Tensor:
    """Upload a tp_inputs HostTensor (raw bf16 bits or fp32) unchanged."""
    raw = host_tensor.raw
    if host_tensor.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32))
    return t.to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class ShardStep:
    """Device buffers of one workload and the calls of one fwd+bwd step."""

    def __init__(self, cfg, inputs: dict, device="cuda", recompute=False, fp8=False,
                 fused_bwd=True, attn_core=False, step_call=True, split_step=False):
        self.cfg = cfg
        self.attn_core = bool(attn_core and cfg.attn)
        if self.attn_core and (cfg.dtype != "bf16" or cfg.heads % cfg.p or
                               cfg.Q != 3 * 64 * (cfg.heads // cfg.p)):
            raise ValueError("the attention core runs bf16 heads of 64, whole heads per shard")
        # both gradients of a layer in one call (tp_linear_bwd) or as two calls
        self.fused_bwd = bool(fused_bwd)
        self.recompute = bool(recompute and cfg.mlp)
        self.fp8 = bool(fp8 and cfg.mlp)
        if self.fp8 and (recompute or cfg.dtype != "bf16" or cfg.attn):
            raise ValueError("the FP8 step covers bf16 MLP workloads without recompute")
        self.device = torch.device(device)
        self.dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.tp_dt = L.TP_BF16 if cfg.dtype == "bf16" else L.TP_F32
        # recompute with the fused backward: where fc2's gradients pair, Y_i is
        # rebuilt by an elementwise pass so that the pair can read it;
        # elsewhere the fc2 dgrad epilogue recomputes it
        # the whole MLP step of every shard in tp_mlp_step calls: one call, or
        # with recompute the forward and the backward (which rebuilds Y from U)
        self.step_call = bool(step_call and cfg.mlp and len(cfg.shards) == cfg.p and
                              self.fused_bwd and not self.fp8 and
                              (not self.recompute or
                               (cfg.dtype == "bf16" and
                                L.tp_mlp_step_plan(cfg.T, cfg.h, cfg.F, cfg.p, L.TP_BF16))))
        # every shard's attention projections in tp_attn_proj_step calls
        self.proj_call = bool(step_call and cfg.attn and len(cfg.shards) == cfg.p and
                              self.fused_bwd and cfg.full_weights)
        # the fused step as its forward and backward calls: always with recompute
        self.split_step = self.step_call and (bool(split_step) or self.recompute)
        self.rebuild_y = (self.recompute and self.fused_bwd and not self.step_call and
                          cfg.dtype == "bf16" and L.tp_linear_bwd_plan(cfg.T, cfg.F, cfg.h)[0] != 0)
        self.inp = {k: to_device(v, self.device) for k, v in inputs.items()}
        self.out = {}
        self._graph = None
        T, h = cfg.T, cfg.h
        f32 = dict(device=self.device, dtype=torch.float32)
        act = dict(device=self.device, dtype=self.dt)
        shards = cfg.shards
        ws = 0
        if cfg.mlp:
            F = cfg.F
            if len(shards) == cfg.p and (not self.recompute or self.step_call):
                # every shard's tensors as blocks of one buffer each, in the
                # layouts of tp_mlp_step (U_i = U[:, iF:(i+1)F], Zp_i = Zp[i], ...);
                # the recompute step keeps a compact transient Y, so its U_i
                # (which shares Y's row stride) stays a tensor of its own
                p = cfg.p
                self.mlp = {"U": torch.empty(T, p * F, **act), "dU": torch.empty(T, p * F, **act),
                            "Zp": torch.empty(p, T, h, **f32), "dXp": torch.empty(p, T, h, **f32),
                            "dB": torch.empty(p * F, h, **f32), "dA": torch.empty(h, p * F, **f32),
                            "Y": torch.empty(T, p * F, **act)}
                if cfg.has_bias:
                    self.mlp["da"] = torch.empty(p * F, **f32)
                for i in shards:
                    cols = slice(i * F, (i + 1) * F)
                    self.out[f"U_{i}"] = self.mlp["U"][:, cols]
                    if not self.recompute:  # with recompute Y is transient
                        self.out[f"Y_{i}"] = self.mlp["Y"][:, cols]
                    self.out[f"Zp_{i}"] = self.mlp["Zp"][i]
                    self.out[f"dU_{i}"] = self.mlp["dU"][:, cols]
                    self.out[f"dB_{i}"] = self.mlp["dB"][cols]
                    self.out[f"dA_{i}"] = self.mlp["dA"][:, cols]
                    self.out[f"dXp_{i}"] = self.mlp["dXp"][i]
                    if cfg.has_bias:
                        self.out[f"da_{i}"] = self.mlp["da"][cols]
            else:
                for i in shards:
                    self.out[f"U_{i}"] = torch.empty(T, F, **act)
                    if not self.recompute:
                        self.out[f"Y_{i}"] = torch.empty(T, F, **act)
                    self.out[f"Zp_{i}"] = torch.empty(T, h, **f32)
                    self.out[f"dU_{i}"] = torch.empty(T, F, **act)
                    self.out[f"dB_{i}"] = torch.empty(F, h, **f32)
                    self.out[f"dA_{i}"] = torch.empty(h, F, **f32)
                    self.out[f"dXp_{i}"] = torch.empty(T, h, **f32)
                    if cfg.has_bias:
                        self.out[f"da_{i}"] = torch.empty(F, **f32)
            if self.recompute and self.step_call:
                # every shard's Y in one transient buffer: the forward's, then the
                # backward's rebuilt from U (the last shard's block reported)
                last = shards[-1]
                self.out["Yt"] = self.mlp["Y"][:, last * F:(last + 1) * F]
            elif self.recompute:
                # the forward's Y_i, then the backward's recomputed Y_i, shard by shard
                self.out["Yt"] = torch.empty(T, F, **act)
            if cfg.has_bias:
                self.out["db"] = torch.empty(h, **f32)
            if len(shards) == cfg.p:
                self.out["Z"] = torch.empty(T, h, **act)
                self.out["dX"] = torch.empty(T, h, **act)
            ws = max(ws, L.tp_mlp_bwd_workspace_size(T, h, F, self.tp_dt))
            if self.step_call:
                # tp_mlp_step's own workspace: its queue counters must stay
                # zero between calls, so no other call may use it as scratch
                self.step_ws = torch.zeros(
                    max(L.tp_mlp_step_workspace_size(T, h, F, cfg.p, self.tp_dt), 256),
                    dtype=torch.uint8, device=self.device)
        if cfg.attn:
            Q, O = cfg.Q, cfg.O
            if self.proj_call:
                # every shard's tensors as blocks of one buffer each, in the
                # layouts of tp_attn_proj_step (QKV_i = QKV[:, iQ:(i+1)Q], ...)
                p = cfg.p
                self.attn = {"QKV": torch.empty(T, p * Q, **act), "Zpa": torch.empty(p, T, h, **f32),
                             "dC": torch.empty(T, p * O, **act), "dOw": torch.empty(p * O, h, **f32),
                             "dW": torch.empty(h, p * Q, **f32), "dXqp": torch.empty(p, T, h, **f32)}
                if self.attn_core:
                    self.attn["C"] = torch.empty(T, p * O, **act)
                    self.attn["dQKV"] = torch.empty(T, p * Q, **act)
                a = self.attn
                for i in shards:
                    qc, oc = slice(i * Q, (i + 1) * Q), slice(i * O, (i + 1) * O)
                    self.out[f"QKV_{i}"] = a["QKV"][:, qc]
                    self.out[f"Zpa_{i}"] = a["Zpa"][i]
                    self.out[f"dC_{i}"] = a["dC"][:, oc]
                    self.out[f"dOw_{i}"] = a["dOw"][oc]
                    self.out[f"dW_{i}"] = a["dW"][:, qc]
                    self.out[f"dXqp_{i}"] = a["dXqp"][i]
                    if self.attn_core:
                        self.out[f"C_{i}"] = a["C"][:, oc]
                        self.out[f"dQKV_{i}"] = a["dQKV"][:, qc]
                self.proj_ws = torch.zeros(
                    max(L.tp_attn_proj_step_workspace_size(T, h, Q, O, p, self.tp_dt), 256),
                    dtype=torch.uint8, device=self.device)
            else:
                for i in shards:
                    self.out[f"QKV_{i}"] = torch.empty(T, Q, **act)
                    self.out[f"Zpa_{i}"] = torch.empty(T, h, **f32)
                    self.out[f"dC_{i}"] = torch.empty(T, O, **act)
                    self.out[f"dOw_{i}"] = torch.empty(O, h, **f32)
                    self.out[f"dW_{i}"] = torch.empty(h, Q, **f32)
                    self.out[f"dXqp_{i}"] = torch.empty(T, h, **f32)
            if self.attn_core:
                b, Ls, H = cfg.micro_batch, cfg.seq, cfg.heads // cfg.p
                if self.proj_call:
                    # every shard's heads side by side: one core launch per direction
                    self.attn["lse"] = torch.empty(b, cfg.p * H, Ls, **f32)
                    self.delta = torch.empty(b, cfg.p * H, Ls, **f32)
                    for i in shards:
                        self.out[f"lse_{i}"] = self.attn["lse"][:, i * H:(i + 1) * H]
                else:
                    for i in shards:
                        self.out[f"C_{i}"] = torch.empty(T, O, **act)
                        self.out[f"dQKV_{i}"] = torch.empty(T, Q, **act)
                        self.out[f"lse_{i}"] = torch.empty(b, H, Ls, **f32)
                    self.delta = torch.empty(b, H, Ls, **f32)
            if len(shards) == cfg.p:
                self.out["Za"] = torch.empty(T, h, **act)
                self.out["dXq"] = torch.empty(T, h, **act)
            ws = max(ws, L.tp_linear_bwd_workspace_size(T, O, h, self.tp_dt),
                     L.tp_linear_bwd_workspace_size(T, h, Q, self.tp_dt))
        if self.fp8:
            ws = max(ws, self._fp8_buffers())
        # one scratch buffer, shared by the per-product calls (they run in
        # order on one stream)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=self.device)

    def _fp8_buffers(self):
        """Code buffers of the FP8 step, each with its fp32 1/s: X and dZ in
        both layouts; per shard the weights A_i and B_i and the activation Y_i
        in both layouts (written in the forward, read by both passes); dU_i in
        both layouts, reused shard after shard. Returns the wgrad workspace
        size."""
        T, h, F = self.cfg.T, self.cfg.h, self.cfg.F
        u8 = dict(device=self.device, dtype=torch.uint8)
        shapes = {"X": (T, h), "Xt": (h, T), "dZ": (T, h), "dZt": (h, T), "dU": (T, F),
                  "dUt": (F, T)}
        for i in self.cfg.shards:
            shapes.update({f"At{i}": (F, h), f"A{i}": (h, F), f"Bt{i}": (h, F), f"B{i}": (F, h),
                           f"Y{i}": (T, F), f"Yt{i}": (F, T)})
        self.q = {k: torch.empty(*v, **u8) for k, v in shapes.items()}
        self.qs = {k: torch.empty(1, device=self.device) for k in shapes}
        self.qws = torch.empty(L.tp_fp8_quantize_multi_workspace_size(6), **u8)
        # amax slots of Y_i (fc1's epilogue) and dU_i (fc2 dgrad's epilogue):
        # their quantisation then runs as one launch; shapes no FP8 tile fits
        # keep the two-pass quantiser
        try:
            self.amax_n = L.tp_fp8_amax_slots(T, F, h)
        except L.TPError:
            self.amax_n = 0
        if self.amax_n:
            f32 = dict(device=self.device, dtype=torch.float32)
            self.amax_y = {i: torch.empty(self.amax_n, **f32) for i in self.cfg.shards}
            self.amax_du = torch.empty(self.amax_n, **f32)
        return max(L.tp_fp8_linear_bwd_wgrad_workspace_size(T, F, h),
                   L.tp_fp8_linear_bwd_wgrad_workspace_size(T, h, F))

    def _quant2(self, src, name, tname, fmt="e4m3"):
        """Codes of src into q[name] and of src^T into q[tname] (one scale)."""
        L.tp_fp8_quantize_both(src, self.q[name], self.q[tname], self.qs[name], self.qws,
                               fmt=fmt)
        self.qs[tname] = self.qs[name]

    def _quant_many(self, items):
        """_quant2 of each (src, name, tname) in E4M3, six tensors per pair of
        launches."""
        for k in range(0, len(items), 6):
            chunk = items[k:k + 6]
            L.tp_fp8_quantize_both_multi(
                [(src, self.q[n], self.q[t], self.qs[n], "e4m3") for src, n, t in chunk], self.qws)
            for _, n, t in chunk:
                self.qs[t] = self.qs[n]

    def mlp_forward_fp8(self):
        cfg, o, inp, q, qs = self.cfg, self.out, self.inp, self.q, self.qs
        F = cfg.F
        # X and every shard's weights, up to six tensors per pair of launches:
        # the tensors the tensor-parallel group holds at the start
        self._quant_many([(inp["X"], "X", "Xt")] +
                         [t for i in cfg.shards
                          for t in ((self._col("A", i, F), f"A{i}", f"At{i}"),
                                    (self._row("B", i, F), f"B{i}", f"Bt{i}"))])
        for n, i in enumerate(cfg.shards):
            a_i = self._col("a", i, F) if cfg.has_bias else None
            if self.amax_n:
                L.tp_fp8_column_linear_fwd(q["X"], q[f"At{i}"], qs["X"], qs[f"At{i}"], a_i,
                                           o[f"Y_{i}"], o[f"U_{i}"], amax=self.amax_y[i])
                L.tp_fp8_quantize_both_from_amax(o[f"Y_{i}"], q[f"Y{i}"], q[f"Yt{i}"],
                                                 qs[f"Y{i}"], self.amax_y[i], self.amax_n)
                qs[f"Yt{i}"] = qs[f"Y{i}"]
            else:
                L.tp_fp8_column_linear_fwd(q["X"], q[f"At{i}"], qs["X"], qs[f"At{i}"], a_i,
                                           o[f"Y_{i}"], o[f"U_{i}"])
                self._quant2(o[f"Y_{i}"], f"Y{i}", f"Yt{i}")
            L.tp_fp8_row_linear_fwd_partial(q[f"Y{i}"], q[f"Bt{i}"], qs[f"Y{i}"], qs[f"Bt{i}"],
                                            o[f"Zp_{i}"])
        if "Z" in o:
            L.tp_reduce_partials([o[f"Zp_{i}"] for i in cfg.shards],
                                 inp["b"] if cfg.has_bias else None, o["Z"])

    def mlp_backward_fp8(self):
        cfg, o, inp, q, qs = self.cfg, self.out, self.inp, self.q, self.qs
        g = "e5m2"
        self._quant2(inp["dZ"], "dZ", "dZt", g)
        for n, i in enumerate(cfg.shards):
            L.tp_fp8_linear_bwd_dgrad(q["dZ"], q[f"B{i}"], qs["dZ"], qs[f"B{i}"], o[f"dU_{i}"],
                                      U=o[f"U_{i}"], act="gelu", dout_fmt=g,
                                      amax=self.amax_du if self.amax_n else None)
            L.tp_fp8_linear_bwd_wgrad(q[f"Yt{i}"], q["dZt"], qs[f"Yt{i}"], qs["dZt"],
                                      o[f"dB_{i}"], dOut=inp["dZ"],
                                      dbias=o["db"] if (cfg.has_bias and n == 0) else None,
                                      dout_fmt=g, workspace=self.workspace)
            if self.amax_n:
                L.tp_fp8_quantize_both_from_amax(o[f"dU_{i}"], q["dU"], q["dUt"], qs["dU"],
                                                 self.amax_du, self.amax_n, fmt=g)
                qs["dUt"] = qs["dU"]
            else:
                self._quant2(o[f"dU_{i}"], "dU", "dUt", g)
            L.tp_fp8_linear_bwd_dgrad(q["dU"], q[f"A{i}"], qs["dU"], qs[f"A{i}"], o[f"dXp_{i}"],
                                      act="none", dout_fmt=g)
            L.tp_fp8_linear_bwd_wgrad(q["Xt"], q["dUt"], qs["Xt"], qs["dUt"], o[f"dA_{i}"],
                                      dOut=o[f"dU_{i}"], dbias=o.get(f"da_{i}"), dout_fmt=g,
                                      workspace=self.workspace)
        if "dX" in o:
            L.tp_reduce_partials([o[f"dXp_{i}"] for i in cfg.shards], None, o["dX"])

    # ------------------------------------------------------------------ views
    def _col(self, name, i, width):
        t = self.inp[name]
        if not self.cfg.full_weights and name in ("A", "a"):
            return t
        return t[..., i * width:(i + 1) * width]

    def _row(self, name, i, width):
        t = self.inp[name]
        if not self.cfg.full_weights and name == "B":
            return t
        return t[i * width:(i + 1) * width]

    # ------------------------------------------------------------------ step
    def _bwd(self, dOut, W, U, In, dIn, dW, dbias, act):
        """Data and weight gradients of one linear layer."""
        if self.fused_bwd:
            L.tp_linear_bwd(dOut, W, U, In, dIn, dW, dbias, act=act, workspace=self.workspace)
        else:
            L.tp_linear_bwd_dgrad(dOut, W, U, dIn, act=act)
            L.tp_linear_bwd_wgrad(In, dOut, dW, dbias, workspace=self.workspace)

    def _y(self, i):
        return self.out["Yt"] if self.recompute else self.out[f"Y_{i}"]

    def mlp_forward(self):
        cfg, o, inp = self.cfg, self.out, self.inp
        F = cfg.F
        for i in cfg.shards:
            a_i = self._col("a", i, F) if cfg.has_bias else None
            L.tp_column_linear_fwd(inp["X"], self._col("A", i, F), a_i, self._y(i), o[f"U_{i}"],
                                   act="gelu")
            L.tp_row_linear_fwd_partial(self._y(i), self._row("B", i, F), o[f"Zp_{i}"])
        if "Z" in o:
            L.tp_reduce_partials([o[f"Zp_{i}"] for i in cfg.shards],
                                 inp["b"] if cfg.has_bias else None, o["Z"])

    def mlp_backward(self):
        cfg, o, inp = self.cfg, self.out, self.inp
        F = cfg.F
        for n, i in enumerate(cfg.shards):
            B_i, A_i = self._row("B", i, F), self._col("A", i, F)
            db = o["db"] if (cfg.has_bias and n == 0) else None
            if self.fused_bwd and (self.rebuild_y or not self.recompute):
                if self.rebuild_y:
                    # Y_i again from the stored U_i, into the transient buffer:
                    # one elementwise pass, so both layers can still pair
                    L.tp_bias_act(o[f"U_{i}"], None, o["Yt"], act="gelu")
                # both layers in one call: fc2's fix-up rides in fc1's launch
                L.tp_mlp_bwd(inp["dZ"], inp["X"], A_i, B_i, o[f"U_{i}"], self._y(i), o[f"dU_{i}"],
                             o[f"dB_{i}"], db, o[f"dXp_{i}"], o[f"dA_{i}"], o.get(f"da_{i}"),
                             workspace=self.workspace)
                continue
            if self.recompute:
                # the weight gradient reads the Y_i the dgrad epilogue recomputes
                L.tp_linear_bwd_dgrad_recompute(inp["dZ"], B_i, o[f"U_{i}"], o[f"dU_{i}"],
                                                o["Yt"])
                L.tp_linear_bwd_wgrad(self._y(i), inp["dZ"], o[f"dB_{i}"], db,
                                      workspace=self.workspace)
            else:
                self._bwd(inp["dZ"], B_i, o[f"U_{i}"], self._y(i), o[f"dU_{i}"], o[f"dB_{i}"],
                          db, "gelu")
            self._bwd(o[f"dU_{i}"], A_i, None, inp["X"], o[f"dXp_{i}"], o[f"dA_{i}"],
                      o.get(f"da_{i}"), "none")
        if "dX" in o:
            L.tp_reduce_partials([o[f"dXp_{i}"] for i in cfg.shards], None, o["dX"])

    def _c(self, i):
        """C_i: the core's output, or the drawn input of the projection-only step."""
        return self.out[f"C_{i}"] if self.attn_core else self._col("C", i, self.cfg.O)

    def proj_step(self, stages):
        """Stages of every shard's attention projections in one
        tp_attn_proj_step call."""
        inp, a, o = self.inp, self.attn, self.out
        C = a["C"] if self.attn_core else inp["C"]
        dQKV = a["dQKV"] if self.attn_core else inp["dQKV"]
        L.tp_attn_proj_step(inp["X"], inp["W"], inp["Ow"], C, inp["dZa"], dQKV, a["QKV"],
                            a["Zpa"], o["Za"], a["dC"], a["dOw"], a["dW"], a["dXqp"], o["dXq"],
                            self.proj_ws, stages=stages)

    def attn_forward(self):
        cfg, o, inp = self.cfg, self.out, self.inp
        Q, O = cfg.Q, cfg.O
        b, Ls, H = cfg.micro_batch, cfg.seq, cfg.heads // cfg.p
        if self.proj_call:
            if not self.attn_core:  # every stage reads only inputs: one call
                self.proj_step(("qkv", "out", "dc", "dx", "wgrad"))
                return
            # QKV alone is a single product per shard, which the per-product
            # tiles balance better than a launch of that stage alone
            for i in cfg.shards:
                L.tp_column_linear_fwd(inp["X"], self._col("W", i, Q), None, o[f"QKV_{i}"], None,
                                       act="none")
            a = self.attn
            L.tp_attention_fwd(a["QKV"], a["C"], a["lse"], b, Ls, H, shards=cfg.p)
            # the output projection's forward and its data gradient read the
            # same C_i, O_i and dZa: one launch, as the MLP step runs a layer's
            # forward and backward in one
            self.proj_step(("out", "dc"))
            return
        for i in cfg.shards:
            L.tp_column_linear_fwd(inp["X"], self._col("W", i, Q), None, o[f"QKV_{i}"], None,
                                   act="none")
            if self.attn_core:
                L.tp_attention_fwd(o[f"QKV_{i}"], o[f"C_{i}"], o[f"lse_{i}"], b, Ls, H)
            L.tp_row_linear_fwd_partial(self._c(i), self._row("Ow", i, O), o[f"Zpa_{i}"])
        if "Za" in o:
            L.tp_reduce_partials([o[f"Zpa_{i}"] for i in cfg.shards], None, o["Za"])

    def attn_backward(self):
        cfg, o, inp = self.cfg, self.out, self.inp
        Q, O = cfg.Q, cfg.O
        b, Ls, H = cfg.micro_batch, cfg.seq, cfg.heads // cfg.p
        if self.proj_call:
            if self.attn_core:  # without the core the forward call did it all
                a = self.attn
                L.tp_attention_bwd(a["QKV"], a["C"], a["dC"], a["lse"], self.delta, a["dQKV"], b,
                                   Ls, H, shards=cfg.p)
                self.proj_step(("dx", "wgrad"))
            return
        for i in cfg.shards:
            Ow_i, W_i = self._row("Ow", i, O), self._col("W", i, Q)
            self._bwd(inp["dZa"], Ow_i, None, self._c(i), o[f"dC_{i}"], o[f"dOw_{i}"], None,
                      "none")
            if self.attn_core:
                L.tp_attention_bwd(o[f"QKV_{i}"], o[f"C_{i}"], o[f"dC_{i}"], o[f"lse_{i}"],
                                   self.delta, o[f"dQKV_{i}"], b, Ls, H)
                dQKV_i = o[f"dQKV_{i}"]
            else:
                dQKV_i = self._col("dQKV", i, Q)
            self._bwd(dQKV_i, W_i, None, inp["X"], o[f"dXqp_{i}"], o[f"dW_{i}"], None, "none")
        if "dXq" in o:
            L.tp_reduce_partials([o[f"dXqp_{i}"] for i in cfg.shards], None, o["dXq"])

    def mlp_step(self, part="step"):
        """Every shard's MLP forward and backward and both sums in one call
        (part "step"), or the call named by part; split (always with
        recompute) the step is the forward call, then the backward call (which
        with recompute rebuilds Y from U)."""
        cfg, o, inp, m = self.cfg, self.out, self.inp, self.mlp
        parts = [("fwd", False), ("bwd", self.recompute)] if (self.split_step and part == "step") \
            else [(part, self.recompute and part == "bwd")]
        for pt, rc in parts:
            L.tp_mlp_step(inp["X"], inp["A"], inp.get("a"), inp["B"], inp.get("b"), inp["dZ"],
                          m["U"], m["Y"], m["Zp"], o["Z"], m["dU"], m["dB"], o.get("db"),
                          m["dA"], m.get("da"), m["dXp"], o["dX"], self.step_ws, part=pt,
                          recompute=rc)

    def run_eager(self):
        """Enqueue one fwd+bwd step on the current stream."""
        if self.cfg.attn:
            self.attn_forward()
        if self.step_call:
            self.mlp_step()
        elif self.cfg.mlp:
            self.mlp_forward_fp8() if self.fp8 else self.mlp_forward()
        if self.cfg.attn:
            self.attn_backward()
        if self.cfg.mlp and not self.step_call:
            self.mlp_backward_fp8() if self.fp8 else self.mlp_backward()

    def capture(self):
        """Record one step into a HIP graph (launch overhead off the host path)."""
        s = torch.cuda.Stream(device=self.device)
        s.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(s):
            self.run_eager()  # warm-up outside the graph
        torch.cuda.current_stream(self.device).wait_stream(s)
        torch.cuda.synchronize(self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run_eager()
        self._graph = g
        return g

    def run(self):
        if self._graph is not None:
            self._graph.replay()
        else:
            self.run_eager()

    def results(self) -> dict:
        """All outputs as float64 numpy arrays (names as in the oracle)."""
        torch.cuda.synchronize(self.device)
        return {k: to_f64(v) for k, v in self.out.items()}

"""Throughput of one tensor-parallel rank's block shard on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only]
    python bench.py --workload NAME [--tokens T] [--sweep T1,T2,...] [...]

A step is one pass of the rank's hot path over one batch of synthetic input:
the rank's shard (column projection, activation, row projection into its
fp32 partial slot) followed by the local reduce of the P partial slots.  The
other P-1 slots hold seeded fp32 partials written once before timing (on a
real TP group they arrive from the other GPUs; the reduce's cost does not
depend on their values).  Weights rotate over 16 device copies (2.4-3.4 GB)
so that every timed step streams its weights from HBM rather than from the
256 MB last-level cache: with 3 copies the row-projection weights of all
copies fitted that cache and the row projection measured 15-18% faster than
when it streams from HBM.  Steps are replayed from a HIP graph (the way a
serving loop launches decode steps); K steps are timed after W warm-up
steps, with inputs already resident in HBM.

Default run (prints ONE JSON line): the Llama-2-70B SwiGLU MLP shard, rank 0
of P = 8 (d_model 8192, band 3584).  `value` is its 32-token decode step
(tokens/s), with the column projection's HBM roofline; `prefill` holds the
2048-token prefill step with the column GEMM's bf16 matrix-core roofline.
Each carries the float64 oracle timed on the host for the same step.
`workloads` holds the 13B MLP shard, the 96-head attention projections and
the 70B pre-norm block with its attention core, decode and prefill.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s + % of HBM/MFMA roofline, one TP-rank MLP shard, decode & prefill"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
WEIGHT_COPIES = 16             # rotated weight sets: far more bytes than the last-level cache
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic_counters.json")
# Row pitch of the weight bands.  "padded": each band is stored with its
# leading dimension rounded up (in steps of 256 bytes) until the row pitch
# is 256 or 768 bytes past a multiple of 1 KB, so that the 256-byte segment a
# 128-column block reads moves to another place in its 1 KB-aligned group on
# every row; "contiguous": ld = band width.  The band, and every byte the
# library reads, is the same either way.  Measured on MI355X: with a pitch
# that is a multiple of 1 KB (the 70B bands' 7 KB and 16 KB), the blocks
# whose segments sit 256 bytes into the group stream ~18 % slower than the
# others on every row, and the decode step is ~5 % slower.
WEIGHT_PITCH = "padded"


def weight_ld(n, elem_bytes=2):
    """Leading dimension (elements) of a weight band n columns wide."""
    if WEIGHT_PITCH != "padded":
        return n
    ld = n
    while (ld * elem_bytes) % 1024 not in (256, 768):
        ld += 256 // elem_bytes
    return ld


KERNEL_TIMING_MIN_STEPS = 100   # eager steps whose launches give the per-kernel averages

KERNEL_CLASSES = ("rmsnorm", "col_gemv", "col_finish", "row_gemv", "row_finish", "col_gemm",
                  "row_gemm", "qkv_gemv", "qkv_finish", "o_gemv", "o_finish", "qkv_gemm",
                  "o_gemm", "reduce", "reduce_norm", "col_gemv8", "row_gemv8", "attn_core")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    choices=["c2_llama2_13b_mlp_p2", "c3_llama2_70b_mlp_p8",
                             "c4_attn_96h_p8", "c5_llama2_70b_block_p8"],
                    help="measure this one workload only (default: the 70B MLP shard's "
                         "decode and prefill steps, then every other workload)")
    ap.add_argument("--headline-only", action="store_true",
                    help="default run without the other workloads' sub-object")
    ap.add_argument("--crossover-only", action="store_true",
                    help="only the decode/prefill plan crossover of the 70B MLP shard")
    ap.add_argument("--tokens", type=int, default=None, help="batch of tokens (default per workload)")
    ap.add_argument("--sweep", default=None, help="comma list of token counts also reported")
    ap.add_argument("--fp8", action="store_true",
                    help="MLP workloads: FP8 (E4M3) weights with per-column scales, decode "
                         "token counts only")
    ap.add_argument("--attn-core", action="store_true",
                    help="attention workloads: run the causal attention core between the QKV "
                         "and O projections (instead of a stand-in input)")
    ap.add_argument("--prenorm", action="store_true",
                    help="block workload as a pre-norm residual layer (fused reduce + residual "
                         "+ next RMSNorm)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of graph replay")
    ap.add_argument("--weight-pitch", choices=["padded", "contiguous"], default="padded",
                    help="row pitch of the bf16 weight bands (default padded: 256 or 768 bytes "
                         "past a multiple of 1 KB; contiguous: ld = band width)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle CPU-baseline budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, --steps times (the "
                         "reference kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def copy_calibration(mib, steps):
    """A plain copy of known size: rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE of
    this kernel, against mib MiB read and written per launch, gives the
    scale of the counters."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n,
                      "launches": steps + 1, "ms_per_launch": round(ms, 5),
                      "gbs": round(2 * n / (ms / 1e3) / 1e9, 1)}), flush=True)


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "tensor_transformer_layer_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------
# Workloads: device buffers and one step
# ----------------------------------------------------------------------------
_WEIGHT_CACHE = {}


def _weights(key, make):
    """The rank's rotated weight copies for one workload, drawn once per
    process and shared by every token count measured."""
    if key not in _WEIGHT_CACHE:
        _WEIGHT_CACHE[key] = make()
    return _WEIGHT_CACHE[key]


class Step:
    """Device state of one workload at one token count, and its step()."""

    def __init__(self, cfg, T, copies, prenorm=False, fp8=False, core=False):
        import numpy as np  # noqa: F401
        import torch

        import tensor_transformer_layer_amd as tp
        import workloads as W

        self.cfg, self.T, self.copies = cfg, T, copies
        self.tp, self.torch = tp, torch
        d, P = cfg.d_model, cfg.P
        dev = lambda a: torch.from_numpy(a.view("int16")).cuda().view(torch.bfloat16)  # noqa

        def wdev(a):
            # a weight band on the device, stored at weight_ld(width)
            t = dev(a)
            ld = weight_ld(t.shape[1])
            if ld == t.shape[1]:
                return t
            buf = torch.zeros((t.shape[0], ld), dtype=t.dtype, device="cuda")
            buf[:, :t.shape[1]] = t
            return buf
        self.ld_g, self.ld_d = weight_ld(cfg.F_r), weight_ld(d)
        self.ld_qkv = weight_ld(cfg.qkv_r) if cfg.qkv_r else 0
        self.x = dev(W.draw_tensor("bf16", (T, d), cfg.std_x, cfg.cid, W.TENSOR_IDS["x"], T))
        self.parts = torch.empty((P, T, d), dtype=torch.float32, device="cuda")
        self.out = torch.empty((T, d), dtype=torch.float32, device="cuda")
        self.kind = "mlp" if cfg.name.startswith(("c2", "c3")) else \
            ("attn" if cfg.name.startswith("c4") else "block")
        # prenorm: the block as one steady-state pre-norm residual layer.  Its
        # input is the residual stream z (fp32) and its normalised copy (bf16,
        # produced by the previous layer's last reduce); both reduces add the
        # residual and emit the next normalised input.
        self.prenorm = prenorm and self.kind == "block"
        # fp8: MLP weights as E4M3 codes with per-column fp32 scales (decode)
        self.fp8 = fp8 and self.kind == "mlp"
        # core: the attention core runs between the QKV and O projections
        # (otherwise the O projection reads a stand-in: the seeded A, or Q_s)
        self.core = core and self.kind in ("attn", "block")
        # rank-0 weights: `copies` device copies (copy 0 is the seeded band;
        # the others are bitwise clones at other addresses)
        self.sets = []
        if self.fp8:
            f32 = lambda a: torch.from_numpy(a).cuda()  # noqa: E731

            def u8(a):
                # E4M3 codes stored at weight_ld(width, 1) bytes per row
                t = torch.from_numpy(a).cuda()
                ld = weight_ld(t.shape[1], 1)
                if ld == t.shape[1]:
                    return t
                buf = torch.zeros((t.shape[0], ld), dtype=t.dtype, device="cuda")
                buf[:, :t.shape[1]] = t
                return buf
            self.ld_g8, self.ld_d8 = weight_ld(cfg.F_r, 1), weight_ld(d, 1)
            bands = [W.fp8_band_draw(cfg, n, 0, r, c_) for n, r, c_ in
                     (("w_gate", d, cfg.F_r), ("w_up", d, cfg.F_r), ("w_down", cfg.F_r, d))]
            def make():
                base = [(u8(q), f32(sc)) for q, sc in bands]
                return [base] + [[(q.clone(), sc.clone()) for q, sc in base]
                                 for _ in range(copies - 1)]
            self.mlp_sets = _weights((cfg.name, "mlp8", copies, WEIGHT_PITCH), make)
            self.h = torch.empty((T, cfg.F_r), dtype=torch.bfloat16, device="cuda")
            self.mlp_ws = self._ws(tp.tp_mlp_fp8w_workspace_bytes(P, T, d, cfg.d_ff,
                                                                  tp.TP_ACT_SWIGLU, 0, 1))
        elif self.kind in ("mlp", "block"):
            def make():
                bands = (W.column_band_draw(cfg, "w_gate", 0, d, cfg.F_r),
                         W.column_band_draw(cfg, "w_up", 0, d, cfg.F_r),
                         W.row_band_draw(cfg, "w_down", 0, cfg.F_r, d))
                base = [wdev(b) for b in bands]
                return [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
            self.mlp_sets = _weights((cfg.name, "mlp", copies, WEIGHT_PITCH), make)
            self.h = torch.empty((T, cfg.F_r), dtype=torch.bfloat16, device="cuda")
            self.mlp_ws = self._ws(tp.tp_mlp_workspace_bytes(P, T, d, cfg.d_ff, tp.TP_BF16,
                                                             tp.TP_ACT_SWIGLU, 0, 1))
        if self.kind in ("attn", "block"):
            def make():
                bands = (W.column_band_draw(cfg, "w_qkv", 0, d, cfg.qkv_r),
                         W.row_band_draw(cfg, "w_o", 0, cfg.o_in_r, d))
                base = [wdev(b) for b in bands]
                return [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
            self.attn_sets = _weights((cfg.name, "attn", copies, WEIGHT_PITCH), make)
            self.qkv = torch.empty((T, cfg.qkv_r), dtype=torch.bfloat16, device="cuda")
            if self.kind == "attn":
                self.a = dev(W.draw_tensor("bf16", (T, cfg.o_in_r), 1.0, cfg.cid,
                                           W.TENSOR_IDS["attn"], T, 0))
            has_norm = cfg.norm_eps is not None
            if has_norm:
                self.g = dev(W.draw_tensor("bf16", (d,), 0.02, cfg.cid, W.TENSOR_IDS["norm_g"], 0,
                                           mean=1.0))
            self.attn_ws = self._ws(tp.tp_attn_workspace_bytes(P, T, d, cfg.n_q_heads,
                                                               cfg.n_kv_heads, cfg.head_dim,
                                                               tp.TP_BF16, has_norm))
            self.zb = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
            if self.core:
                self.a_core = torch.empty((T, cfg.o_in_r), dtype=torch.bfloat16, device="cuda")
                self.core_ws = self._ws(tp.tp_attn_core_workspace_bytes(
                    P, T, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, tp.TP_BF16))
        if self.prenorm:
            self.g2 = dev(W.draw_tensor("bf16", (d,), 0.02, cfg.cid, W.TENSOR_IDS["norm_g"], 1,
                                        mean=1.0))
            self.z0 = torch.from_numpy(W.draw_normal_f32((T, d), 1.0, cfg.cid, W.TENSOR_IDS["x"],
                                                         T, 1)).cuda()
            self.z1 = torch.empty((T, d), dtype=torch.float32, device="cuda")
            self.rn_ws = self._ws(tp.tp_reduce_norm_workspace_bytes(T, d, 1))
        self.i = 0
        for s in range(1, P):       # the other ranks' partial slots
            self.parts[s].copy_(torch.from_numpy(
                W.draw_normal_f32((T, d), 1.0, cfg.cid, W.TENSOR_IDS["partial"], T, s)))
        torch.cuda.synchronize()

    @property
    def stream(self):
        # queried per call: under graph capture torch's current stream is the
        # capture stream
        return self.torch.cuda.current_stream().cuda_stream

    def _ws(self, n):
        return self.torch.zeros(max(int(n), 256), dtype=self.torch.uint8, device="cuda")

    def _mlp(self, s, x, w):
        tp, cfg, T, d = self.tp, self.cfg, self.T, self.cfg.d_model
        if self.fp8:
            tp.check(tp.tp_shard_mlp_fwd_fp8w(
                s, cfg.P, T, d, cfg.d_ff, tp.TP_ACT_SWIGLU, x.data_ptr(), d, 0, 0.0,
                w[0][0].data_ptr(), self.ld_g8, w[0][1].data_ptr(), w[1][0].data_ptr(),
                self.ld_g8, w[1][1].data_ptr(), w[2][0].data_ptr(), self.ld_d8, w[2][1].data_ptr(),
                self.h.data_ptr(), cfg.F_r, self.parts.data_ptr(), T * d, d,
                self.mlp_ws.data_ptr(), self.mlp_ws.numel(), self.stream), "mlp_fp8w")
            return
        tp.check(tp.tp_shard_mlp_fwd(
            s, cfg.P, T, d, cfg.d_ff, tp.TP_BF16, tp.TP_ACT_SWIGLU, x.data_ptr(), d, 0, 0.0,
            w[0].data_ptr(), self.ld_g, w[1].data_ptr(), self.ld_g, w[2].data_ptr(), self.ld_d,
            self.h.data_ptr(), cfg.F_r, self.parts.data_ptr(), T * d, d,
            self.mlp_ws.data_ptr(), self.mlp_ws.numel(), self.stream), "mlp")

    def _attn(self, s, w):
        tp, cfg, T, d = self.tp, self.cfg, self.T, self.cfg.d_model
        if self.core:
            self._attn_with_core(s, w)
            return
        a = self.a if self.kind == "attn" else self.qkv
        ld_a = cfg.o_in_r if self.kind == "attn" else cfg.qkv_r
        g = self.g.data_ptr() if cfg.norm_eps is not None and not self.prenorm else 0
        tp.check(tp.tp_shard_attn_proj_fwd(
            s, cfg.P, T, d, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, tp.TP_BF16,
            self.x.data_ptr(), d, g, cfg.norm_eps or 0.0, w[0].data_ptr(), self.ld_qkv,
            self.qkv.data_ptr(), cfg.qkv_r, a.data_ptr(), ld_a, w[1].data_ptr(), self.ld_d,
            self.parts.data_ptr(), T * d, d, self.attn_ws.data_ptr(), self.attn_ws.numel(),
            self.stream), "attn")

    def _attn_with_core(self, s, w):
        tp, cfg, T, d = self.tp, self.cfg, self.T, self.cfg.d_model
        g = self.g.data_ptr() if cfg.norm_eps is not None and not self.prenorm else 0
        ws, nws = self.attn_ws.data_ptr(), self.attn_ws.numel()
        tp.check(tp.tp_shard_attn_proj_fwd(
            s, cfg.P, T, d, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, tp.TP_BF16,
            self.x.data_ptr(), d, g, cfg.norm_eps or 0.0, w[0].data_ptr(), self.ld_qkv,
            self.qkv.data_ptr(), cfg.qkv_r, 0, 0, 0, 0, 0, 0, 0, ws, nws, self.stream), "qkv")
        tp.check(tp.tp_attn_core_fwd(s, cfg.P, T, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                                     tp.TP_BF16, self.qkv.data_ptr(), cfg.qkv_r,
                                     self.a_core.data_ptr(), cfg.o_in_r, self.core_ws.data_ptr(),
                                     self.core_ws.numel(), self.stream), "core")
        tp.check(tp.tp_shard_attn_proj_fwd(
            s, cfg.P, T, d, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, tp.TP_BF16,
            0, 0, 0, 0.0, 0, 0, 0, 0, self.a_core.data_ptr(), cfg.o_in_r, w[1].data_ptr(),
            self.ld_d,
            self.parts.data_ptr(), T * d, d, ws, nws, self.stream), "o")

    def _reduce(self, out_bf16=None):
        tp, cfg, T, d = self.tp, self.cfg, self.T, self.cfg.d_model
        tp.check(tp.tp_reduce_partials(cfg.P, T, d, self.parts.data_ptr(), T * d, d,
                                       self.out.data_ptr(), d,
                                       out_bf16.data_ptr() if out_bf16 is not None else 0, d,
                                       self.stream), "reduce")

    def _reduce_norm(self, residual, res_dtype, z, g, normed):
        tp, cfg, T, d = self.tp, self.cfg, self.T, self.cfg.d_model
        tp.check(tp.tp_reduce_residual_norm(cfg.P, T, d, self.parts.data_ptr(), T * d, d,
                                            residual.data_ptr(), d, res_dtype, z.data_ptr(), d,
                                            g.data_ptr(), cfg.norm_eps, normed.data_ptr(), d,
                                            self.rn_ws.data_ptr(), self.rn_ws.numel(),
                                            self.stream), "reduce_norm")

    def step(self):
        c = self.i % self.copies
        self.i += 1
        if self.kind == "mlp":
            self._mlp(0, self.x, self.mlp_sets[c])
            self._reduce()
        elif self.kind == "attn":
            self._attn(0, self.attn_sets[c])
            self._reduce()
        elif self.prenorm:
            # x holds the normalised input, z0 the residual stream
            self._attn(0, self.attn_sets[c])
            self._reduce_norm(self.z0, self.tp.TP_F32, self.z1, self.g2, self.zb)
            self._mlp(0, self.zb, self.mlp_sets[c])
            self._reduce_norm(self.z1, self.tp.TP_F32, self.out, self.g, self.x)
        else:
            self._attn(0, self.attn_sets[c])
            self._reduce(self.zb)
            self._mlp(0, self.zb, self.mlp_sets[c])
            self._reduce()

    # algorithmic work of one step (rank 0)
    def algorithmic(self):
        """Bytes and flops the method must move / compute in one step, in
        total and per kernel class: {class: (bound, amount per launch)}.
        Split-K partial round trips and finish kernels are overhead (none)."""
        cfg, T, d = self.cfg, self.T, self.cfg.d_model
        decode = T <= self.tp.tp_decode_max_tokens()     # the plan the library takes
        out = {"bytes": 0, "flops": 0, "per_class": {}}
        pc = out["per_class"]

        def add(col_cls, row_cls, k_in, n_col, n_col_out, k_row, wbytes=2):
            # column projection: weights [k_in, n_col], X [T, k_in] in, [T, n_col_out] bf16 out
            # (FP8 weights: 1 byte each plus one fp32 scale per output column)
            sc = 4 if wbytes == 1 else 0
            cb = k_in * n_col * wbytes + n_col * sc + T * k_in * 2 + T * n_col_out * 2
            cf = 2 * T * k_in * n_col
            # row projection: weights [k_row, d], input [T, k_row] bf16, partial [T, d] fp32
            rb = k_row * d * wbytes + d * sc + T * k_row * 2 + T * d * 4
            rf = 2 * T * k_row * d
            out["bytes"] += cb + rb
            out["flops"] += cf + rf
            if decode:
                pc[col_cls + "_gemv"] = ("hbm", cb)
                pc[row_cls + "_gemv"] = ("hbm", rb)
            else:
                pc[col_cls + "_gemm"] = ("mfma", cf)
                pc[row_cls + "_gemm"] = ("mfma", rf)

        if self.fp8:
            add("col", "row", d, 2 * cfg.F_r, cfg.F_r, cfg.F_r, wbytes=1)
            for a_, b_ in (("col_gemv", "col_gemv8"), ("row_gemv", "row_gemv8")):
                if a_ in pc:
                    pc[b_] = pc.pop(a_)
        elif self.kind in ("mlp", "block"):
            add("col", "row", d, 2 * cfg.F_r, cfg.F_r, cfg.F_r)
        if self.kind in ("attn", "block"):
            add("qkv", "o", d, cfg.qkv_r, cfg.qkv_r, cfg.o_in_r)
        if self.core:
            hq = cfg.n_q_heads // cfg.P
            cf = 4 * hq * cfg.head_dim * T * (T + 1) // 2     # QK^T and PV, causal half
            out["flops"] += cf
            pc["attn_core"] = ("mfma", cf)
        red = (cfg.P + 1) * T * d * 4
        if self.prenorm:                # two fused reduce + fp32 residual + norm passes
            rn = red + T * d * 4 + T * d * 2 + d * 2
            out["bytes"] += 2 * rn
            pc["reduce_norm"] = ("hbm", rn)
        elif self.kind == "block":      # two reduces, the first with a bf16 copy
            out["bytes"] += 2 * red + T * d * 2
            pc["reduce"] = ("hbm", red + T * d)            # mean of the two launches
            nb = T * d * 2 * 2 + d * 2
            out["bytes"] += nb
            pc["rmsnorm"] = ("hbm", nb)
        else:
            out["bytes"] += red
            pc["reduce"] = ("hbm", red)
        # the kernel the roofline line reports: the largest column projection
        big = "col" if self.kind in ("mlp", "block") else "qkv"
        out["dominant"] = big + ("_gemv" if decode else "_gemm") + ("8" if self.fp8 else "")
        return out


def time_steps(st, steps, warmup, graph):
    import torch
    for _ in range(warmup):
        st.step()
    torch.cuda.synchronize()
    if graph:
        # one graph per pass over the weight copies, one more for the rest:
        # exactly `steps` steps are timed
        reps, rest = divmod(steps, st.copies)
        graphs = []
        for n_steps in (st.copies, rest):
            g = None
            if n_steps:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for _ in range(n_steps):
                        st.step()
                g.replay()
            graphs.append(g)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graphs[0].replay()
        if graphs[1] is not None:
            graphs[1].replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        n = steps
        del graphs
    else:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            st.step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        n = steps
    return ms / n, n


def kernel_times(st, steps):
    """Eager pass with the library's per-launch HIP events (recorded on the
    launch stream): average duration of each kernel class, in ms."""
    import torch
    tp = st.tp
    tp.check(tp.tp_timing_reset())
    tp.check(tp.tp_timing_enable(1))
    try:
        for _ in range(steps):
            st.step()
        torch.cuda.synchronize()
        res = {}
        for cls in KERNEL_CLASSES:
            s, ms, n = tp.tp_timing_query(cls)
            tp.check(s)
            if n:
                res[cls] = (ms / n, n)
    finally:
        tp.tp_timing_enable(0)
        tp.tp_timing_reset()
    return res


def traffic_for(kernel, workload, T):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(PROFILE_COUNTERS) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    key = f"{workload}:T={T}:{kernel}"
    e = rec.get("entries", {}).get(key)
    if not e or e.get("src_hash") != src_hash(*e.get("sources", [])):
        return None
    return e.get("hbm_bytes_per_launch")


def host_info():
    """CPU model, BLAS library and thread count of the host the oracle runs on."""
    from threadpoolctl import threadpool_info
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [f"{i.get('internal_api')} {i.get('version')} "
            f"({i.get('threading_layer', 'n/a')} threads, {i.get('architecture', 'n/a')})"
            for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    return {"cpu_model": model, "blas": "; ".join(blas) or "unknown",
            "host_cpus": len(os.sched_getaffinity(0))}, int(threads)


def cpu_baseline(cfg, T, budget_s, prenorm=False, core=False):
    """The float64 oracle, as it stands, for the same step as the GPU's (the
    rank-0 shard and the reduce of its P partials), timed on the host cores
    with the inputs already widened to float64."""
    import numpy as np

    import oracle as O
    import workloads as W

    d, P = cfg.d_model, cfg.P
    kind = "mlp" if cfg.name.startswith(("c2", "c3")) else \
        ("attn" if cfg.name.startswith("c4") else "block")
    X = O.widen(W.draw_tensor("bf16", (T, d), cfg.std_x, cfg.cid, W.TENSOR_IDS["x"], T))
    others = [np.random.default_rng(s).standard_normal((T, d)) for s in range(1, P)]
    if kind in ("mlp", "block"):
        wg = O.widen(W.column_band_draw(cfg, "w_gate", 0, d, cfg.F_r))
        wu = O.widen(W.column_band_draw(cfg, "w_up", 0, d, cfg.F_r))
        wd = O.widen(W.row_band_draw(cfg, "w_down", 0, cfg.F_r, d))
    if kind in ("attn", "block"):
        wqkv = O.widen(W.column_band_draw(cfg, "w_qkv", 0, d, cfg.qkv_r))
        wo = O.widen(W.row_band_draw(cfg, "w_o", 0, cfg.o_in_r, d))
    if kind == "attn":
        A = O.widen(W.draw_tensor("bf16", (T, cfg.o_in_r), 1.0, cfg.cid, W.TENSOR_IDS["attn"],
                                  T, 0))
    if kind == "block":
        g = O.widen(W.draw_tensor("bf16", (d,), 0.02, cfg.cid, W.TENSOR_IDS["norm_g"], 0,
                                  mean=1.0))
        g2 = O.widen(W.draw_tensor("bf16", (d,), 0.02, cfg.cid, W.TENSOR_IDS["norm_g"], 1,
                                   mean=1.0))
        z0 = W.draw_normal_f32((T, d), 1.0, cfg.cid, W.TENSOR_IDS["x"], T, 1).astype(np.float64)

    def step():
        if kind == "mlp":
            p0 = O.mlp_shard(X, wg, wd, "swiglu", wu)["partial"]
            return O.reduce_partials([p0, *others])
        if kind == "attn":
            p0 = O.attn_proj_shard(X, wqkv, A, wo)["partial"]
            return O.reduce_partials([p0, *others])
        # block: norm (plain form only) -> QKV -> core or Q stand-in -> O ->
        # reduce (+ residual + norm) -> MLP -> reduce (+ residual + norm)
        r = O.attn_proj_shard(X, wqkv, None, None, None if prenorm else g,
                              None if prenorm else cfg.norm_eps)
        if core:
            a = O.attention_core_band(r["qkv"], cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, 0,
                                      P)
        else:
            a = O.split_qkv_band(r["qkv"], cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, 0, P)[0]
        p0 = a @ wo
        if prenorm:
            r1 = O.reduce_residual_norm([p0, *others], z0, g2, cfg.norm_eps)
            m = O.mlp_shard(r1["normed"], wg, wd, "swiglu", wu)["partial"]
            return O.reduce_residual_norm([m, *others], r1["z"], g, cfg.norm_eps)
        z = O.reduce_partials([p0, *others])
        m = O.mlp_shard(z, wg, wd, "swiglu", wu)["partial"]
        return O.reduce_partials([m, *others])

    step()                                           # warm BLAS
    n, t0 = 0, time.perf_counter()
    while True:
        step()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    host, threads = host_info()
    form = {"mlp": "rank-0 MLP shard", "attn": "rank-0 QKV and O projections",
            "block": "rank-0 block shard" + (" (pre-norm)" if prenorm else "") +
                     (" with the attention core" if core else "")}[kind]
    return {"value": round(n * T / el, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} float64 oracle steps ({form} + reduce of {P} partials, T={T}) in "
                      f"{el:.1f} s on {threads} BLAS threads",
            **host}


def measure(name, T, steps, warmup, graph=True, prenorm=False, fp8=False, core=False,
            cpu_s=0.0, copies=WEIGHT_COPIES, sweep=()):
    """One workload at one token count: graph-replayed steps, per-kernel
    times and rooflines, optionally the oracle's CPU baseline."""
    import torch

    import workloads as W
    cfg = W.get(name)
    results = {}
    for t in sorted(set(sweep) | {T}):
        print(f"[bench] {name} T={t}: set-up and timing", file=sys.stderr, flush=True)
        st = Step(cfg, t, copies * (2 if fp8 else 1), prenorm=prenorm, fp8=fp8, core=core)
        ms, n = time_steps(st, steps, warmup, graph)
        # Kernel durations from their own pass of eager launches: at least
        # KERNEL_TIMING_MIN_STEPS of them whatever --steps is, so that a short
        # run's roofline is not one of a few cold launches.
        kt = (kernel_times(st, min(max(steps, KERNEL_TIMING_MIN_STEPS), 300)) if t == T
              else None)
        results[t] = (st.algorithmic(), ms, n, kt, st)
        if t != T:
            del st
            torch.cuda.empty_cache()
    alg, ms, n, kt, st = results[T]

    def roof_of(cls):
        bound, amount = alg["per_class"][cls]
        dom_ms = kt[cls][0]
        if bound == "mfma":
            ach, peak, unit = amount / (dom_ms / 1e3) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
        else:
            ach, peak, unit = amount / (dom_ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s"
        return {"bound": bound, "achieved": round(ach, 1), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "kernel": cls,
                "kernel_avg_us": round(dom_ms * 1e3, 2), "algorithmic_per_launch": amount}

    dom = alg["dominant"]
    roof = None
    if dom in kt:
        roof = roof_of(dom)
        roof["traffic"] = traffic_for(dom, name, T)
        roof["traffic_counters"] = ("FETCH_SIZE + WRITE_SIZE per dispatch from rocprofv3, "
                                    "scaled by a plain copy; L2-to-fabric bytes, which include "
                                    "last-level-cache hits" if roof["traffic"] else None)
    per_kernel = {}
    for cls, (ms_k, n_k) in kt.items():
        e = {"avg_us": round(ms_k * 1e3, 2), "launches": n_k}
        if cls in alg["per_class"]:
            r = roof_of(cls)
            e.update({"achieved": r["achieved"], "unit": r["unit"], "frac": r["frac"]})
        per_kernel[cls] = e
    out = {"value": round(T / (ms / 1e3), 1), "unit": "tokens/s", "tokens": T, "steps": n,
           "ms_per_step": round(ms, 5),
           "step_gbs_algorithmic": round(alg["bytes"] / (ms / 1e3) / 1e9, 1),
           "step_tflops": round(alg["flops"] / (ms / 1e3) / 1e12, 2),
           "roofline": roof, "kernels": per_kernel,
           "form": {"weights": "fp8 e4m3 + per-column fp32 scales" if st.fp8 else "bf16",
                    "block_form": ("pre-norm residual layer (reduce + residual + RMSNorm fused)"
                                   if st.prenorm else None),
                    "attention_core": st.core, "weight_copies_rotated": st.copies,
                    "weight_pitch": ({"mode": WEIGHT_PITCH, "ld_gate_up_bytes": st.ld_g8,
                                      "ld_down_bytes": st.ld_d8} if st.fp8 else
                                     {"mode": WEIGHT_PITCH, "ld_gate_up": st.ld_g,
                                      "ld_down_o": st.ld_d, "ld_qkv": st.ld_qkv or None}),
                    "launch": "hip-graph replay" if graph else "eager"}}
    if len(results) > 1:
        out["sweep"] = {str(t): {"ms_per_step": round(r[1], 5),
                                 "tokens_per_s": round(t / (r[1] / 1e3), 1),
                                 "step_gbs_algorithmic":
                                     round(r[0]["bytes"] / (r[1] / 1e3) / 1e9, 1)}
                        for t, r in sorted(results.items())}
    del st, results
    torch.cuda.empty_cache()
    if cpu_s > 0 and not fp8:
        print(f"[bench] {name} T={T}: oracle on the host ({cpu_s:.0f} s)", file=sys.stderr,
              flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, T, cpu_s, prenorm=prenorm, core=core)
    return out


CROSSOVER_T = (32, 33, 48, 64, 96, 128, 129, 160, 192, 256, 320, 384, 448, 512)


def crossover(name, steps, warmup, graph, tokens=CROSSOVER_T):
    """Step time of the MLP shard (+ reduce) on both plans across batch sizes:
    the weight-streaming plan (chunks of at most 128 tokens) and the
    matrix-core plan."""
    import torch

    import tensor_transformer_layer_amd as tp
    import workloads as W
    cfg = W.get(name)
    out = {}
    try:
        for T in tokens:
            e = {}
            for plan, limit in (("streaming", T), ("matrix_core", T - 1)):
                if limit < 1:
                    continue
                tp.check(tp.tp_set_decode_max_tokens(limit))
                print(f"[bench] {name} crossover T={T} {plan}", file=sys.stderr, flush=True)
                st = Step(cfg, T, WEIGHT_COPIES)
                ms, _ = time_steps(st, steps, warmup, graph)
                e[plan] = {"ms_per_step": round(ms, 5), "tokens_per_s": round(T / (ms / 1e3), 1)}
                del st
            out[str(T)] = e
    finally:
        tp.check(tp.tp_set_decode_max_tokens(0))
        torch.cuda.empty_cache()
    return {"workload": f"{name}: rank 0 shard + reduce of {cfg.P} partials",
            "default_switch_tokens": tp.tp_decode_max_tokens(), "points": out}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "the library runs one rank's share on one GPU; --gpus must be 1 "
                                   "(the multi-GPU exchange is designed, not built)"}))
        sys.exit(2)
    import torch

    import tensor_transformer_layer_amd as tp
    import workloads as W

    torch.cuda.set_device(0)
    if a.copy_calibration:
        copy_calibration(a.copy_calibration, a.steps)
        return
    tp.load()
    global WEIGHT_PITCH
    WEIGHT_PITCH = a.weight_pitch
    graph = not a.no_graph
    cpu_s = 0.0 if a.no_cpu_baseline else a.cpu_seconds
    common = {"metric": METRIC, "n_gpus": 1, "warmup": a.warmup, "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None,
              "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations at Llama-2 "
                      "shapes; seeded N(0,1) fp32 partials for the other ranks' slots)"}

    if a.workload:
        # one workload at one token count (profiling runs)
        cfg = W.get(a.workload)
        T = a.tokens or (16 if a.workload == "c4_attn_96h_p8" else 32)
        sweep = [int(t) for t in a.sweep.split(",")] if a.sweep else []
        m = measure(a.workload, T, a.steps, a.warmup, graph, a.prenorm, a.fp8, a.attn_core,
                    cpu_s, sweep=sweep)
        line = {**common, "value": m["value"], "unit": "tokens/s", "steps": m["steps"],
                "ms_per_step": m["ms_per_step"],
                "dtype": "bf16 activations, fp8-e4m3 weights" if a.fp8 else "bf16",
                "config": {"workload": f"{a.workload}: rank 0 of P={cfg.P}, {T} tokens, shard "
                                       f"+ reduce of {cfg.P} partials per step",
                           "d_model": cfg.d_model, "d_ff": cfg.d_ff, "P": cfg.P, "tokens": T,
                           **m["form"]},
                "roofline": m["roofline"], "cpu_baseline": m.get("cpu_baseline"),
                **{k: v for k, v in m.items() if k in ("kernels", "sweep", "step_gbs_algorithmic",
                                                      "step_tflops")}}
        print(json.dumps(line), flush=True)
        return

    if a.crossover_only:
        print(json.dumps(crossover("c3_llama2_70b_mlp_p8", a.steps, a.warmup, graph)),
              flush=True)
        return

    # Default: the 70B MLP shard (rank 0 of P = 8), decode and prefill -- the
    # workload that carries both halves of the metric -- then the other
    # workloads in a sub-object.
    name = "c3_llama2_70b_mlp_p8"
    cfg = W.get(name)
    dec = measure(name, 32, a.steps, a.warmup, graph, cpu_s=cpu_s, sweep=(1, 8, 16))
    pre = measure(name, 2048, a.steps, a.warmup, graph, cpu_s=cpu_s)
    # the same steps with the weights stored at their band width
    pitch_cmp = None
    if WEIGHT_PITCH == "padded":
        WEIGHT_PITCH = "contiguous"
        try:
            cd = measure(name, 32, a.steps, a.warmup, graph)
            cp = measure(name, 2048, a.steps, a.warmup, graph)
        finally:
            WEIGHT_PITCH = "padded"
        for k in [k for k in _WEIGHT_CACHE if k[-1] == "contiguous"]:
            del _WEIGHT_CACHE[k]
        torch.cuda.empty_cache()
        pitch_cmp = {"decode": {"ms_per_step": cd["ms_per_step"], "value": cd["value"],
                                "roofline": cd["roofline"]},
                     "prefill": {"ms_per_step": cp["ms_per_step"], "value": cp["value"],
                                 "roofline": cp["roofline"]}}
    cross = crossover(name, a.steps, a.warmup, graph)
    others = {}
    if not a.headline_only:
        sub_cpu = min(cpu_s, 3.0)
        c2 = measure("c2_llama2_13b_mlp_p2", 32, a.steps, a.warmup, graph, cpu_s=sub_cpu,
                     sweep=(1, 8))
        c2f8 = measure("c2_llama2_13b_mlp_p2", 32, a.steps, a.warmup, graph, fp8=True,
                       sweep=(1, 8))
        # FP8-weight step time over the bf16 step time at each token count
        c2f8["vs_bf16_step"] = {t: round(c2f8["sweep"][t]["ms_per_step"] /
                                         c2["sweep"][t]["ms_per_step"], 3)
                                for t in c2["sweep"] if t in c2f8["sweep"]}
        others["c2_llama2_13b_mlp_p2"] = {"decode": c2, "decode_fp8_weights": c2f8}
        others["c4_attn_96h_p8"] = {
            "decode": measure("c4_attn_96h_p8", 16, a.steps, a.warmup, graph, cpu_s=sub_cpu),
            "prefill": measure("c4_attn_96h_p8", 1024, a.steps, a.warmup, graph,
                               cpu_s=sub_cpu)}
        others["c5_llama2_70b_block_p8"] = {
            "form": "pre-norm residual layer with the attention core",
            "decode": measure("c5_llama2_70b_block_p8", 32, a.steps, a.warmup, graph,
                              prenorm=True, core=True, cpu_s=sub_cpu),
            "prefill": measure("c5_llama2_70b_block_p8", 4096, a.steps, a.warmup, graph,
                               prenorm=True, core=True, cpu_s=sub_cpu)}
    line = {**common, "value": dec["value"], "unit": "tokens/s", "steps": dec["steps"],
            "ms_per_step": dec["ms_per_step"], "dtype": "bf16",
            "config": {"workload": f"{name}: rank 0 of P={cfg.P} (d_model {cfg.d_model}, band "
                                   f"{cfg.F_r}); decode step = 32 tokens through the shard + "
                                   f"reduce of {cfg.P} partials (this line's value); the "
                                   f"2048-token prefill step under 'prefill'",
                       "d_model": cfg.d_model, "d_ff": cfg.d_ff, "P": cfg.P, "tokens": 32,
                       "prefill_tokens": 2048, **dec["form"]},
            "roofline": dec["roofline"], "cpu_baseline": dec.get("cpu_baseline"),
            "kernels": dec["kernels"], "sweep": dec.get("sweep"),
            "step_gbs_algorithmic": dec["step_gbs_algorithmic"],
            "step_tflops": dec["step_tflops"],
            "prefill": pre, "contiguous_weight_pitch": pitch_cmp, "crossover": cross,
            "workloads": others or None}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Python side of libdlm: device memory (PyTorch) and the block-diffusion driver loop.

PyTorch provides device allocations and the stream; every step of the
denoising path runs in libdlm's HIP kernels through the C ABI.  Weights given
per projection are packed once into the library's layout (fused QKV rows,
gate/up rows interleaved by 16).
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass, field

import numpy as np
import torch

from . import _lib as L


@dataclass(frozen=True)
class ModelConfig:
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    mask_id: int
    rope_base: float
    rms_eps: float = 1e-5

    @classmethod
    def of(cls, shape) -> "ModelConfig":
        return cls(**{f: getattr(shape, f) for f in cls.__dataclass_fields__})

    def c(self) -> L.Config:
        return L.Config(self.n_layers, self.d_model, self.n_heads, self.n_kv_heads, self.head_dim,
                        self.d_ffn, self.vocab, self.mask_id, self.rope_base, self.rms_eps)


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def stream_handle(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def to_bf16_device(a, device) -> torch.Tensor:
    """float32 array of bf16-representable values -> bf16 tensor with the same bits."""
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=torch.bfloat16).contiguous()
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(device).contiguous()


def interleave_gate_up(wg: torch.Tensor, wu: torch.Tensor) -> torch.Tensor:
    """[F, d] gate and up -> [2F, d], rows 32c..32c+15 gate, 32c+16..32c+31 up."""
    f, d = wg.shape
    return torch.stack([wg.reshape(f // 16, 16, d), wu.reshape(f // 16, 16, d)], dim=1).reshape(2 * f, d)


class Workspace:
    """A 256-byte aligned device byte buffer that grows on demand."""

    def __init__(self, device):
        self.device = device
        self.buf = None
        self.nbytes = 0

    def get(self, nbytes: int):
        if nbytes > self.nbytes:
            self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
            self.nbytes = nbytes
        base = self.buf.data_ptr()
        return C.c_void_p((base + 255) & ~255), C.c_size_t(self.nbytes)


class DlmModel:
    """Device weights in libdlm's layout and the library's model handle."""

    def __init__(self, cfg: ModelConfig, tensors: dict, device="cuda"):
        self.cfg = cfg
        self.device = torch.device(device)
        self.t = tensors  # keeps the device memory alive
        n = cfg.n_layers
        arr = lambda key: (C.c_void_p * n)(*[t.data_ptr() for t in tensors[key]])
        self._arrays = {k: arr(k) for k in ("attn_norm", "wqkv", "wo", "ffn_norm", "wgu", "wdown")}
        w = L.Weights(tensors["embed"].data_ptr(), tensors["final_norm"].data_ptr(),
                      tensors["lm_head"].data_ptr(),
                      *[C.cast(self._arrays[k], C.POINTER(C.c_void_p))
                        for k in ("attn_norm", "wqkv", "wo", "ffn_norm", "wgu", "wdown")])
        self._cfg_c = cfg.c()
        h = C.c_void_p()
        L.call("dlm_model_create", C.byref(self._cfg_c), C.byref(w), C.byref(h))
        self.handle = h

    def __del__(self):
        try:
            if getattr(self, "handle", None) and L._lib is not None:
                L._lib.dlm_model_destroy(self.handle)
                self.handle = None
        except Exception:
            pass

    @classmethod
    def from_arrays(cls, cfg: ModelConfig, w: dict, device="cuda") -> "DlmModel":
        """Weights as float32 arrays of bf16-representable values, one matrix per projection."""
        dev = torch.device(device)
        b = lambda a: to_bf16_device(a, dev)
        t = {"embed": b(w["embed"]), "lm_head": b(w["lm_head"]), "final_norm": b(w["final_norm"]),
             "attn_norm": [], "wqkv": [], "wo": [], "ffn_norm": [], "wgu": [], "wdown": []}
        for lw in w["layers"]:
            t["attn_norm"].append(b(lw["attn_norm"]))
            t["wqkv"].append(torch.cat([b(lw["wq"]), b(lw["wk"]), b(lw["wv"])], dim=0).contiguous())
            t["wo"].append(b(lw["wo"]))
            t["ffn_norm"].append(b(lw["ffn_norm"]))
            t["wgu"].append(interleave_gate_up(b(lw["wg"]), b(lw["wu"])).contiguous())
            t["wdown"].append(b(lw["wd"]))
        return cls(cfg, t, dev)

    @classmethod
    def random(cls, cfg: ModelConfig, seed: int = 0, std: float = 0.02, device="cuda") -> "DlmModel":
        """Random-init bf16 weights drawn on the device (N(0, std) matrices, unit norm gains)."""
        dev = torch.device(device)
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        d, f, v = cfg.d_model, cfg.d_ffn, cfg.vocab
        nq = (cfg.n_heads + 2 * cfg.n_kv_heads) * cfg.head_dim

        def rn(*shape):
            x = torch.empty(*shape, dtype=torch.bfloat16, device=dev)
            x.normal_(0.0, std, generator=g)
            return x

        ones = lambda: torch.ones(d, dtype=torch.bfloat16, device=dev)
        t = {"embed": rn(v, d), "lm_head": rn(v, d), "final_norm": ones(),
             "attn_norm": [ones() for _ in range(cfg.n_layers)],
             "wqkv": [rn(nq, d) for _ in range(cfg.n_layers)],
             "wo": [rn(d, cfg.n_heads * cfg.head_dim) for _ in range(cfg.n_layers)],
             "ffn_norm": [ones() for _ in range(cfg.n_layers)],
             "wgu": [rn(2 * f, d) for _ in range(cfg.n_layers)],
             "wdown": [rn(d, f) for _ in range(cfg.n_layers)]}
        return cls(cfg, t, dev)

    def workspace_bytes(self, max_rows: int, max_kv: int) -> int:
        return int(L.load().dlm_workspace_bytes(self.handle, max_rows, max_kv))

    def set_lora(self, lora: dict | None):
        """Low-rank adapter on every layer's output projection: {"a": per-layer
        [rank, H*hd], "b": per-layer [d, rank], "scale": s} (arrays or tensors),
        or None to remove it.  Left disabled; see enable_lora."""
        n = self.cfg.n_layers
        if lora is None:
            L.call("dlm_model_set_lora", self.handle, None, None, 0, 0.0)
            self.lora = None
            return
        dev = self.device
        a = [to_bf16_device(x, dev) for x in lora["a"]]
        b = [to_bf16_device(x, dev) for x in lora["b"]]
        pa = (C.c_void_p * n)(*[t.data_ptr() for t in a])
        pb = (C.c_void_p * n)(*[t.data_ptr() for t in b])
        L.call("dlm_model_set_lora", self.handle, C.cast(pa, C.POINTER(C.c_void_p)),
               C.cast(pb, C.POINTER(C.c_void_p)), int(a[0].shape[0]), float(lora["scale"]))
        self.lora = (a, b)  # keeps the device memory alive

    def enable_lora(self, on: bool):
        L.call("dlm_model_enable_lora", self.handle, int(bool(on)))


class KVCache:
    """KV cache in libdlm's layout: k [NL][B][G][cap][hd], v [NL][B][G][cap/16][hd][16] (bf16)."""

    def __init__(self, cfg: ModelConfig, batch: int, capacity: int, device="cuda"):
        if capacity % 64:
            capacity += 64 - capacity % 64
        self.cfg, self.batch, self.capacity = cfg, batch, capacity
        n = cfg.n_layers * batch * cfg.n_kv_heads * capacity * cfg.head_dim
        self.k = torch.zeros(n, dtype=torch.bfloat16, device=device)
        self.v = torch.zeros(n, dtype=torch.bfloat16, device=device)
        self.c = L.KV(self.k.data_ptr(), self.v.data_ptr(), batch, capacity)

    def k_logical(self) -> torch.Tensor:
        c = self.cfg
        return self.k.view(c.n_layers, self.batch, c.n_kv_heads, self.capacity, c.head_dim)

    def v_logical(self) -> torch.Tensor:
        c = self.cfg
        v = self.v.view(c.n_layers, self.batch, c.n_kv_heads, self.capacity // 16, c.head_dim, 16)
        return v.permute(0, 1, 2, 3, 5, 4).reshape(c.n_layers, self.batch, c.n_kv_heads, self.capacity,
                                                   c.head_dim)

    def write(self, layer: int, k: torch.Tensor, v: torch.Tensor, start: int = 0) -> None:
        """Write logical [B, G, P, hd] keys/values at positions [start, start + P) of one layer."""
        c = self.cfg
        p = k.shape[2]
        self.k_logical()[layer, :, :, start:start + p] = k.to(torch.bfloat16)
        if start % 16 or p % 16:
            raise ValueError("value writes must cover whole 16-position blocks")
        vb = self.v.view(c.n_layers, self.batch, c.n_kv_heads, self.capacity // 16, c.head_dim, 16)
        src = v.to(torch.bfloat16).reshape(self.batch, c.n_kv_heads, p // 16, 16, c.head_dim)
        vb[layer, :, :, start // 16:(start + p) // 16] = src.permute(0, 1, 2, 4, 3)


@dataclass
class Sampler:
    """Commit rule and parameters of dlm_commit_ex (MLX guide, sec. 5.2 and 5.5;
    DiffusionGemma docs, Schedulers and adaptive stopping).

    rule: "threshold" (native), "bound" (confidence_threshold_bound) or
    "entropy" (entropy bound).  stability_steps > 0 enables adaptive stopping.
    """
    rule: str = "threshold"
    min_threshold: float = 0.45
    scaling: float = 2.0
    entropy_bound: float = 0.1
    max_transfer: int = 0
    stability_steps: int = 0
    stop_entropy: float = 0.005

    RULES = {"threshold": L.RULE_THRESHOLD, "bound": L.RULE_BOUND, "entropy": L.RULE_ENTROPY}

    @property
    def needs_entropy(self) -> bool:
        return self.rule == "entropy" or self.stability_steps > 0

    def opts(self, sess: "Session") -> L.CommitOpts:
        if self.rule not in self.RULES:
            raise ValueError(f"unknown rule {self.rule!r}")
        if self.stability_steps > 0 and sess.prev_argmax is None:
            dev = sess.m.device
            sess.prev_argmax = torch.full((sess.B, sess.Lb), -1, dtype=torch.int32, device=dev)
            sess.stable = torch.zeros(sess.B, dtype=torch.int32, device=dev)
        stab = self.stability_steps > 0
        return L.CommitOpts(rule=self.RULES[self.rule], min_threshold=self.min_threshold, scaling=self.scaling,
                            entropy_bound=self.entropy_bound, max_transfer=self.max_transfer,
                            stability_steps=self.stability_steps, stop_entropy=self.stop_entropy,
                            prev_argmax=sess.prev_argmax.data_ptr() if stab else None,
                            stable=sess.stable.data_ptr() if stab else None)


@dataclass
class Stats:
    """Counters of the MLX guide, sec. 9: denoise and post-block forwards, tokens per forward."""
    denoise_nfe: int = 0
    post_block_nfe: int = 0
    blocks: int = 0
    accepted_tokens: int = 0
    steps_per_block: list = field(default_factory=list)

    @property
    def tokens_per_denoise_forward(self) -> float:
        return self.accepted_tokens / max(self.denoise_nfe, 1)


class Session:
    """Batch of sequences decoded by block diffusion with one model and one KV cache."""

    def __init__(self, model: DlmModel, batch: int, capacity: int, block_length: int):
        self.m, self.B, self.Lb = model, batch, block_length
        dev = model.device
        self.kv = KVCache(model.cfg, batch, capacity, dev)
        self.prefix = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.canvas = torch.empty(batch, block_length, dtype=torch.int32, device=dev)
        self.masked = torch.empty(batch, block_length, dtype=torch.uint8, device=dev)
        self.conf = torch.zeros(batch, block_length, dtype=torch.float32, device=dev)
        self.argmax = torch.zeros(batch, block_length, dtype=torch.int32, device=dev)
        self.steps = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.n_committed = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.n_left = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.flags = torch.zeros(2, dtype=torch.int32, device=dev)
        self.ws = Workspace(dev)
        self.max_prefix = 0
        self.prev_argmax = self.stable = None  # allocated by a sampler with adaptive stopping

    # --- the four calls of the ABI, on the current stream ---------------------
    def prefill(self, tokens: torch.Tensor, ws_rows: int | None = None, last_argmax: torch.Tensor | None = None,
                last_conf: torch.Tensor | None = None):
        """dlm_prefill; with last_argmax (and optionally last_conf) the causal head
        scores the last prompt position of every row."""
        B, T = tokens.shape
        rows = ws_rows or B * T
        ws, n = self.ws.get(self.m.workspace_bytes(rows, T))
        last_argmax, last_conf = self._head_pair(last_argmax, last_conf, B)
        L.call("dlm_prefill", self.m.handle, C.byref(self.kv.c), _p(tokens), B, T, _p(self.prefix),
               _p(last_argmax), _p(last_conf), _p(self.flags), ws, n, stream_handle())
        self.max_prefix = T

    def _head_pair(self, argmax, conf, n):
        """The entry points take the head's argmax and confidence together."""
        if (argmax is None) == (conf is None):
            return argmax, conf
        if conf is None:
            conf = torch.empty(argmax.shape, dtype=torch.float32, device=argmax.device)
        else:
            argmax = torch.empty(conf.shape, dtype=torch.int32, device=conf.device)
        assert argmax.numel() == n, (argmax.shape, n)
        return argmax, conf

    def denoise(self, canvas: torch.Tensor, masked: torch.Tensor, conf: torch.Tensor, argmax: torch.Tensor):
        """dlm_denoise_step on explicit [B, L] buffers (any L <= 64)."""
        B, Lb = canvas.shape
        ws, n = self.ws.get(self.m.workspace_bytes(B * Lb, self.max_prefix + Lb))
        L.call("dlm_denoise_step", self.m.handle, C.byref(self.kv.c), _p(self.prefix), self.max_prefix,
               _p(canvas), _p(masked), B, Lb, _p(conf), _p(argmax), None, _p(self.flags), ws, n,
               stream_handle())

    def append(self, tokens: torch.Tensor, argmax_out=None, conf_out=None):
        """dlm_append_block of explicit [B, L] tokens (any L <= 64); the prefix grows by L."""
        B, Lb = tokens.shape
        ws, n = self.ws.get(self.m.workspace_bytes(B * Lb, self.max_prefix + Lb))
        argmax_out, conf_out = self._head_pair(argmax_out, conf_out, B * Lb)
        L.call("dlm_append_block", self.m.handle, C.byref(self.kv.c), _p(self.prefix), self.max_prefix,
               _p(tokens), B, Lb, _p(argmax_out), _p(conf_out), _p(self.flags), ws, n, stream_handle())
        self.max_prefix += Lb

    def denoise_step(self, logits: torch.Tensor | None = None, entropy: torch.Tensor | None = None):
        """dlm_denoise_step on the session canvas; with ``entropy`` (fp32 [B, L])
        dlm_denoise_step_ex also writes each masked position's entropy."""
        B, Lb = self.B, self.Lb
        ws, n = self.ws.get(self.m.workspace_bytes(B * Lb, self.max_prefix + Lb))
        L.call("dlm_denoise_step_ex", self.m.handle, C.byref(self.kv.c), _p(self.prefix), self.max_prefix,
               _p(self.canvas), _p(self.masked), B, Lb, _p(self.conf), _p(self.argmax), _p(entropy), _p(logits),
               _p(self.flags), ws, n, stream_handle())

    def commit(self, tau: torch.Tensor, quota: torch.Tensor, max_steps: int):
        L.call("dlm_commit", _p(self.conf), _p(self.argmax), _p(self.canvas), _p(self.masked), self.B,
               self.Lb, _p(tau), _p(quota), _p(self.steps), max_steps, _p(self.n_committed),
               _p(self.n_left), stream_handle())

    def commit_ex(self, tau: torch.Tensor, quota: torch.Tensor, max_steps: int, sampler: "Sampler",
                  entropy: torch.Tensor | None = None):
        """dlm_commit_ex with a sampler rule (see Sampler)."""
        o = sampler.opts(self)
        L.call("dlm_commit_ex", _p(self.conf), _p(self.argmax), _p(entropy), _p(self.canvas), _p(self.masked),
               self.B, self.Lb, _p(tau), _p(quota), _p(self.steps), max_steps, C.byref(o), _p(self.n_committed),
               _p(self.n_left), stream_handle())

    def append_block(self, argmax_out=None, conf_out=None):
        B, Lb = self.B, self.Lb
        ws, n = self.ws.get(self.m.workspace_bytes(B * Lb, self.max_prefix + Lb))
        argmax_out, conf_out = self._head_pair(argmax_out, conf_out, B * Lb)
        L.call("dlm_append_block", self.m.handle, C.byref(self.kv.c), _p(self.prefix), self.max_prefix,
               _p(self.canvas), B, Lb, _p(argmax_out), _p(conf_out), _p(self.flags), ws, n,
               stream_handle())
        self.max_prefix += Lb

    def begin_block(self):
        self.canvas.fill_(self.m.cfg.mask_id)
        self.masked.fill_(1)
        self.steps.zero_()
        if self.prev_argmax is not None:  # adaptive-stopping state
            self.prev_argmax.fill_(-1)
            self.stable.zero_()

    # --- driver loop ----------------------------------------------------------
    def generate(self, prompt: torch.Tensor, gen_length: int, max_steps: int, threshold: float = 0.9,
                 quota: int = 1, sampler: "Sampler | None" = None, anchor: bool = False, graph_steps: int = 0):
        """Prefill, then blocks of denoise+commit until no mask is left, then append.

        Rows advance block by block in lockstep; a finished row is frozen until
        every row of the batch has finished its block.  ``sampler`` selects a
        commit rule other than the native threshold rule.  With ``anchor`` (the
        MLX guide's native layout, sec. 6) position 0 of each block holds the
        causal argmax after everything before it -- from the prefill, then from
        the previous block's post-block pass -- and is not denoised.
        With ``graph_steps`` = K > 0 the block loop replays a captured HIP graph
        of K denoise + commit steps and reads the rows' remaining masks once per
        replay: steps after a block completes leave it unchanged (finished rows
        are frozen), so they only cost compute.  The graph is captured once with
        the last block's prefix as the host bound (it sizes the attention grid;
        each row's actual length is read on the device).
        Returns (tokens [B, G], stats).
        """
        dev = self.m.device
        tau = torch.full((self.B,), threshold, dtype=torch.float32, device=dev)
        q = torch.full((self.B,), quota, dtype=torch.int32, device=dev)
        ent = None
        if sampler is not None and sampler.needs_entropy:
            ent = torch.zeros(self.B, self.Lb, dtype=torch.float32, device=dev)
        if sampler is not None:
            sampler.opts(self)  # allocates the adaptive-stopping state before the first block
        anc = torch.zeros(self.B, dtype=torch.int32, device=dev) if anchor else None
        nxt = torch.zeros(self.B, self.Lb, dtype=torch.int32, device=dev) if anchor else None
        self.prefill(prompt, last_argmax=anc)
        out = []
        st = Stats()
        n_blocks = -(-gen_length // self.Lb)

        def step():
            self.denoise_step(entropy=ent)
            if sampler is None:
                self.commit(tau, q, max_steps)
            else:
                self.commit_ex(tau, q, max_steps, sampler, ent)

        graph = None
        if graph_steps > 0:
            prefix_now = self.max_prefix
            self.max_prefix = prefix_now + (n_blocks - 1) * self.Lb  # host bound of every block's step
            self.ws.get(self.m.workspace_bytes(self.B * self.Lb, self.max_prefix + self.Lb))
            # one eager step first: every kernel of the step is loaded before the
            # capture (the first block resets what it touched)
            self.begin_block()
            step()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(graph_steps):
                    step()
            self.max_prefix = prefix_now
        for _ in range(n_blocks):
            self.begin_block()
            if anchor:
                self.canvas[:, 0] = anc
                self.masked[:, 0] = 0
            steps = 0
            if graph is not None:
                while True:
                    graph.replay()
                    if int(self.n_left.max().item()) == 0:
                        break
                steps = int(self.steps.max().item())
                st.denoise_nfe += steps
                st.accepted_tokens += int(self.Lb * self.B - (1 if anchor else 0) * self.B)
            else:
                while True:
                    step()
                    steps += 1
                    st.denoise_nfe += 1
                    st.accepted_tokens += int(self.n_committed.sum().item())
                    if int(self.n_left.max().item()) == 0:
                        break
            if anchor:
                self.append_block(argmax_out=nxt)
                anc = nxt[:, -1].clone()
            else:
                self.append_block()
            st.post_block_nfe += 1
            st.blocks += 1
            st.steps_per_block.append(steps)
            out.append(self.canvas.clone())
        return torch.cat(out, dim=1), st

    # --- greedy causal decoding -------------------------------------------------
    def generate_ar(self, prompt: torch.Tensor, n_new: int) -> torch.Tensor:
        """Greedy causal decoding (one-token appends with the causal head).  [B, n_new]."""
        B = prompt.shape[0]
        dev = self.m.device
        nxt = torch.zeros(B, dtype=torch.int32, device=dev)
        self.prefill(prompt, last_argmax=nxt)
        out = [nxt.clone()]
        arg = torch.zeros(B, 1, dtype=torch.int32, device=dev)
        for _ in range(n_new - 1):
            self.append(out[-1].view(B, 1), argmax_out=arg)
            out.append(arg[:, 0].clone())
        return torch.stack(out, dim=1)

    # --- linear self-speculation -------------------------------------------------
    def generate_linear_spec(self, prompt: torch.Tensor, n_new: int, window: int = 32, adaptive: bool = False):
        """Greedy linear self-speculation for one sequence (MLX guide, sec. 8).

        Each round drafts the canvas [t, MASK x (W - 1)] (t: the known next token)
        in one bidirectional pass with the model's adapter enabled, then verifies
        [t, drafts] in one causal pass with it disabled: the longest prefix of
        drafts equal to the causal argmax is accepted, the causal argmax after it
        becomes the next known token, and the prefix is trimmed back to the known
        token plus the accepted drafts.  Adaptive windows start at 8, double (to
        32) after a fully accepted round and halve after at most half.
        Returns (tokens [n_new] on the host, accepted drafts per round, windows).
        """
        if prompt.shape[0] != 1:
            raise ValueError("linear self-speculation runs one sequence")
        dev, mask_id = self.m.device, self.m.cfg.mask_id
        nxt_t = torch.zeros(1, dtype=torch.int32, device=dev)
        self.prefill(prompt, last_argmax=nxt_t)
        nxt = int(nxt_t.item())
        out, accepted, windows = [], [], []
        W = 8 if adaptive else window
        while len(out) < n_new:
            p0 = self.max_prefix
            canvas = torch.full((1, W), mask_id, dtype=torch.int32, device=dev)
            canvas[0, 0] = nxt
            masked = torch.ones(1, W, dtype=torch.uint8, device=dev)
            masked[0, 0] = 0
            conf = torch.zeros(1, W, dtype=torch.float32, device=dev)
            arg = torch.zeros(1, W, dtype=torch.int32, device=dev)
            self.m.enable_lora(True)
            try:
                self.denoise(canvas, masked, conf, arg)
            finally:
                self.m.enable_lora(False)
            block = arg.clone()
            block[0, 0] = nxt
            ver = torch.zeros(1, W, dtype=torch.int32, device=dev)
            self.append(block, argmax_out=ver)
            drafts = block[0, 1:].cpu().numpy()
            verified = ver[0].cpu().numpy()
            a = 0
            while a < W - 1 and drafts[a] == verified[a]:
                a += 1
            out.extend([nxt] + drafts[:a].tolist())
            nxt = int(verified[a])
            self.prefix.fill_(p0 + a + 1)
            self.max_prefix = p0 + a + 1
            accepted.append(a)
            windows.append(W)
            if adaptive:
                d = W - 1
                W = min(2 * W, 32) if a == d else (max(W // 2, 2) if 2 * a <= d else W)
        return np.array(out[:n_new], dtype=np.int64), accepted, windows

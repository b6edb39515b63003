"""A decode session over the C ABI, with torch providing device memory and the stream.

DeviceWeights uploads canonical bf16 weights (uint16 bit arrays) and, for the
fp8, int8 and int4 modes, quantises every Linear matrix on the device with
dar_quantize_fp8_rows / dar_quantize_int8_rows / dar_quantize_int4_groups.
DarSession owns the workspace and the dar_ctx and wraps
prefill / decode_frame with torch tensors. Everything here is marshalling:
pointers, sizes and buffers; the arithmetic runs in libdar.so.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import native as N

LINEAR_SUFFIXES = ("wqkv", "wo", "w1", "w3", "w2")


def _dev(t):
    return ctypes.c_void_p(t.data_ptr())


class DeviceWeights:
    """Device copies of the canonical tensors; quantised modes replace each Linear
    matrix by its codes (fp8, int8: [rows][cols]; int4: packed [rows][cols/2])
    and add its scales (fp8, int8: [rows]; int4: [rows][cols/128])."""

    def __init__(self, dims, host_tensors: dict, wtype: str = "bf16", device="cuda", stream=None,
                 keep_bf16_linears: bool = False):
        self.dims = dims
        self.wtype = wtype
        self.t = {}
        self.scale = {}
        s = stream if stream is not None else torch.cuda.current_stream(device)
        sp = ctypes.c_void_p(s.cuda_stream)
        for name, bits in host_tensors.items():
            arr = np.ascontiguousarray(bits).view(np.int16)
            dev = torch.from_numpy(arr).to(device, non_blocking=False)
            if wtype in ("fp8", "int8", "int4") and self.is_linear(name):
                rows, cols = dev.shape
                if wtype == "int4":
                    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
                    sc = torch.empty((rows, cols // 128), dtype=torch.float32, device=device)
                    quantize = N.dar_quantize_int4_groups
                else:
                    q = torch.empty((rows, cols), dtype=torch.uint8 if wtype == "fp8" else torch.int8, device=device)
                    sc = torch.empty((rows,), dtype=torch.float32, device=device)
                    quantize = N.dar_quantize_fp8_rows if wtype == "fp8" else N.dar_quantize_int8_rows
                with torch.cuda.stream(s):
                    quantize(_dev(dev), rows, cols, _dev(q), _dev(sc), sp)
                self.t[name] = q
                self.scale[name] = sc
                if keep_bf16_linears:
                    self.t[name + ".bf16"] = dev
                else:
                    s.synchronize()
                    del dev
            else:
                self.t[name] = dev
        s.synchronize()

    @staticmethod
    def is_linear(name):
        return name == "fast.head" or name.split(".")[-1] in LINEAR_SUFFIXES

    def ptr(self, name):
        return self.t[name].data_ptr()

    def sptr(self, name):
        return self.scale[name].data_ptr() if name in self.scale else None

    def layer_struct(self, prefix):
        L = N.dar_layer_weights()
        L.attn_norm = self.ptr(f"{prefix}.attn_norm")
        L.ffn_norm = self.ptr(f"{prefix}.ffn_norm")
        for m in LINEAR_SUFFIXES:
            setattr(L, m, self.ptr(f"{prefix}.{m}"))
            setattr(L, f"{m}_scale", self.sptr(f"{prefix}.{m}"))
        return L

    def struct(self):
        d = self.dims
        W = N.dar_weights()
        W.w0 = self.ptr("w0")
        slow = (N.dar_layer_weights * d.n_layers_slow)(*[self.layer_struct(f"slow.{i}") for i in range(d.n_layers_slow)])
        W.slow = slow
        W.slow_final_norm = self.ptr("slow.final_norm")
        keep = [slow]
        if d.n_res > 0:
            emb = (ctypes.c_void_p * d.n_res)(*[self.ptr(f"fast.emb.{k}") for k in range(d.n_res)])
            fast = (N.dar_layer_weights * d.n_layers_fast)(*[self.layer_struct(f"fast.{i}") for i in range(d.n_layers_fast)])
            W.fast_emb = emb
            W.fast = fast
            W.fast_final_norm = self.ptr("fast.final_norm")
            W.fast_head = self.ptr("fast.head")
            W.fast_head_scale = self.sptr("fast.head")
            keep += [emb, fast]
        return W, keep


class DarSession:
    """One dar_ctx: workspace, stream, prefill and frame decode with torch tensors.

    batch > 1 decodes that many sequences in lockstep: prefill takes one
    prompt per sequence, frames and forced codes are [batch][1 + n_res], logits
    [batch][1 + n_res][vmax]. With batch 1 the leading axis is dropped."""

    def __init__(self, dims, weights: DeviceWeights, max_len: int, device="cuda", stream=None, graph=False,
                 batch=1, paging=None):
        self.dims = dims
        self.max_len = max_len
        self.device = device
        self.batch = batch
        self.stream = stream if stream is not None else torch.cuda.Stream(device)
        self.cfg = N.make_config(dims, max_len, weights.wtype, max_batch=batch)
        self.paging = N.dar_paging(*paging) if paging is not None else None
        nbytes = (N.dar_workspace_bytes_paged(self.cfg, self.paging) if self.paging is not None
                  else N.dar_workspace_bytes(self.cfg))
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.weights = weights
        wstruct, self._keep = weights.struct()
        ws, st = ctypes.c_void_p(self.workspace.data_ptr()), ctypes.c_void_p(self.stream.cuda_stream)
        if self.paging is not None:
            self.ctx = N.dar_create_paged(self.cfg, self.paging, wstruct, ws, nbytes, st)
        else:
            self.ctx = N.dar_create(self.cfg, wstruct, ws, nbytes, st)
        self._seq_toks = {}
        N.dar_set_graph(self.ctx, graph)
        self.fc = dims.n_res + 1
        self.vmax = max(dims.vocab_c0, dims.vocab_res if dims.n_res > 0 else 0)
        self.codes = torch.zeros(batch, self.fc, dtype=torch.int32, device=device)
        self.logits = torch.zeros(batch, self.fc, self.vmax, dtype=torch.float32, device=device)
        self.forced = torch.zeros(batch, self.fc, dtype=torch.int32, device=device)
        # these fills run on torch's stream; the context writes the buffers on its own
        torch.cuda.current_stream(device).synchronize()

    def close(self):
        if self.ctx:
            N.dar_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _forced_ptr(self, forced):
        if forced is None:
            return None
        f = torch.as_tensor(np.asarray(forced, dtype=np.int32).reshape(self.batch, self.fc))
        with torch.cuda.stream(self.stream):
            self.forced.copy_(f.to(self.device, non_blocking=False))
        return _dev(self.forced)

    def prefill(self, tokens, forced=None, want=True):
        prompts = [tokens] if self.batch == 1 else list(tokens)
        lens = [len(p) for p in prompts]
        toks = torch.as_tensor(np.concatenate([np.asarray(p, dtype=np.int32) for p in prompts])).to(self.device)
        torch.cuda.current_stream(self.device).synchronize()
        fp = self._forced_ptr(forced)
        N.dar_prefill(self.ctx, self.batch, _dev(toks), lens, fp, _dev(self.codes) if want else None,
                      _dev(self.logits) if want else None)
        self._toks = toks
        return self._out(want)

    def seq_add(self, slot, tokens):
        """Paged context: prefill one prompt into a free slot; its frame 0
        comes out of the next decode_frame."""
        toks = torch.as_tensor(np.asarray(tokens, dtype=np.int32)).to(self.device)
        torch.cuda.current_stream(self.device).synchronize()
        N.dar_seq_add(self.ctx, slot, _dev(toks), len(tokens))
        self._seq_toks[slot] = toks  # read on the stream: kept until the slot is reused

    def seq_remove(self, slot):
        N.dar_seq_remove(self.ctx, slot)

    def pages_free(self):
        return N.dar_pages_free(self.ctx)

    def decode_frame(self, forced=None, want=True):
        fp = self._forced_ptr(forced)
        N.dar_decode_frame(self.ctx, fp, _dev(self.codes) if want else None, _dev(self.logits) if want else None)
        return self._out(want)

    def _out(self, want):
        if not want:
            return None
        self.stream.synchronize()
        codes, logits = self.codes.cpu().numpy().copy(), self.logits.cpu().numpy().copy()
        return (codes[0], logits[0]) if self.batch == 1 else (codes, logits)

    def ring(self, first, count):
        dst = torch.empty(count, self.batch, self.fc, dtype=torch.int32, device=self.device)
        # the copy runs on the context's stream: nothing queued on torch's may touch dst after it
        torch.cuda.current_stream(self.device).synchronize()
        N.dar_codes(self.ctx, first, count, _dev(dst))
        self.stream.synchronize()
        out = dst.cpu().numpy()
        return out[:, 0] if self.batch == 1 else out

    def position(self):
        pos = N.dar_position(self.ctx, self.batch)
        return pos[0] if self.batch == 1 else list(pos)

    def reset(self):
        N.dar_reset(self.ctx)

    def set_graph(self, enable):
        N.dar_set_graph(self.ctx, enable)

    def nonfinite(self):
        return N.dar_nonfinite(self.ctx)

    def set_sampling(self, temperature=None, top_k=None, top_p=1.0, penalty=1.0, window=0, uniforms=None):
        """Sample the codes (uniforms: [max_len][batch][1 + n_res] values in
        [0, 1), kept on the device while the session samples); no arguments:
        greedy argmax again."""
        if temperature is None:
            N.dar_set_sampling(self.ctx, None)
            self._uniforms = None
            return
        u = torch.as_tensor(np.asarray(uniforms, dtype=np.float32).reshape(self.max_len, self.batch, self.fc))
        self._uniforms = u.to(self.device).contiguous()
        torch.cuda.current_stream(self.device).synchronize()
        N.dar_set_sampling(self.ctx, N.make_sampling(temperature, top_k, top_p, penalty, window,
                                                     self._uniforms.data_ptr()))

    def time_kind(self, kind):
        N.dar_time_kind(self.ctx, kind)

    def kind_time(self):
        return N.dar_kind_time(self.ctx)

    def profile_frame(self):
        return N.dar_profile_frame(self.ctx)


class CodecSession:
    """One dar_codec context: device copies of the canonical codec tensors
    (uint16 bf16 bit arrays by name), its workspace and stream, and
    decode(codes) -> audio with torch tensors. Marshalling only."""

    def __init__(self, dims, host: dict, max_frames: int, device="cuda", stream=None):
        self.dims = dims
        self.device = device
        self.max_frames = max_frames
        self.stream = stream if stream is not None else torch.cuda.Stream(device)
        self.t = {name: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).to(device)
                  for name, v in host.items()}
        ptr = lambda name: ctypes.c_void_p(self.t[name].data_ptr())  # noqa: E731
        self.cfg = N.make_codec_config(dims, max_frames)
        nbytes = N.dar_codec_workspace_bytes(self.cfg)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        tables = (ctypes.c_void_p * dims.n_codebooks)(*[ptr(f"codec.rvq.{k}").value for k in range(dims.n_codebooks)])
        blocks = (N.dar_codec_block * len(dims.rates))()
        for i in range(len(dims.rates)):
            p = f"codec.b{i}"
            blocks[i].alpha, blocks[i].up_w, blocks[i].up_b = ptr(f"{p}.alpha"), ptr(f"{p}.up.w"), ptr(f"{p}.up.b")
            for j in range(len(dims.dilations)):
                r = f"{p}.ru{j}"
                u = blocks[i].units[j]
                u.alpha1, u.w1, u.b1 = ptr(f"{r}.alpha1"), ptr(f"{r}.w1"), ptr(f"{r}.b1")
                u.alpha2, u.w2, u.b2 = ptr(f"{r}.alpha2"), ptr(f"{r}.w2"), ptr(f"{r}.b2")
        w = N.dar_codec_weights(ctypes.cast(tables, ctypes.POINTER(ctypes.c_void_p)), ptr("codec.in.w"),
                                ptr("codec.in.b"), ctypes.cast(blocks, ctypes.POINTER(N.dar_codec_block)),
                                ptr("codec.out.alpha"), ptr("codec.out.w"), ptr("codec.out.b"))
        self._keep = (tables, blocks)
        # the uploads ran on torch's stream; the context reads them on its own
        torch.cuda.current_stream(device).synchronize()
        self.ctx = N.dar_codec_create(self.cfg, w, ctypes.c_void_p(self.workspace.data_ptr()), nbytes,
                                      ctypes.c_void_p(self.stream.cuda_stream))
        self.codes = torch.zeros(max_frames, dims.n_codebooks, dtype=torch.int32, device=device)
        self.audio = torch.zeros(max_frames * dims.hop, dtype=torch.float32, device=device)
        torch.cuda.current_stream(device).synchronize()

    def load_codes(self, codes):
        """Copy host codes [frames][n_codebooks] to the device buffer; returns frames."""
        c = torch.as_tensor(np.ascontiguousarray(codes, dtype=np.int32))
        n = c.shape[0]
        with torch.cuda.stream(self.stream):
            self.codes[:n].copy_(c.to(self.device))
        return n

    def decode(self, codes=None, frames=None, want=True):
        """Decode `codes` (host) or, with codes None, the first `frames` frames
        already in the device buffer; returns the audio as a host array."""
        n = self.load_codes(codes) if codes is not None else frames
        N.dar_codec_decode(self.ctx, ctypes.c_void_p(self.codes.data_ptr()), n, ctypes.c_void_p(self.audio.data_ptr()))
        if not want:
            return None
        self.stream.synchronize()
        return self.audio[:n * self.dims.hop].cpu().numpy().copy()

    def profile(self, frames):
        return N.dar_codec_profile(self.ctx, ctypes.c_void_p(self.codes.data_ptr()), frames,
                                   ctypes.c_void_p(self.audio.data_ptr()))

    def anomalies(self):
        return N.dar_codec_anomalies(self.ctx)

    def close(self):
        if getattr(self, "ctx", None):
            N.dar_codec_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

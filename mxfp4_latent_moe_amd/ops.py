"""Torch-facing wrappers of the C-ABI calls (the five of the layer, the capped
routing, the REAP saliency and the combine with REAP fused in), and a layer object that chains the layer's calls on one stream.  Argument marshalling only: tensors are passed as
device pointers, the stream as its HIP handle; all compute runs in the HIP
library."""
from __future__ import annotations

import torch

from . import _lib
from ._lib import (MOE_DT_BF16, MOE_DT_BF16X2, MOE_DT_F32, MOE_FN_COMBINE_NORM_UP, MOE_FN_GROUPED_GEMM,
                   MOE_FN_PERMUTE, MOE_FN_ROUTE, MOE_FN_SHARED_FFN, MOE_OP_DOWN,
                   MOE_OP_GATEUP_SITU, MOE_OP_GATEUP_SITU_BF16X2, MoeShape, check, load)


def _p(t):
    return None if t is None else t.data_ptr()


def _s(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def shape_of(ls, operand_mode: int = _lib.MOE_OPND_BF16X2, beta=4.0, beta_lin=25.0, rms_eps=1e-6) -> MoeShape:
    """MoeShape from any object with the LayerShape fields."""
    return _lib.make_shape(ls.hidden, ls.latent, ls.n_experts, ls.top_k, ls.inter, ls.n_shared,
                           ls.shared_inter, beta, beta_lin, rms_eps, operand_mode)


def workspace_bytes(shape: MoeShape, fn: int, n: int) -> int:
    return int(load().moe_workspace_bytes(shape, fn, n))


def route(shape, x, w_router, bias, w_down, topk_ids, topk_w, z, gap, ws, stream=None):
    check("moe_route", load().moe_route(shape, x.shape[0], _p(x), _p(w_router), _p(bias), _p(w_down),
                                        _p(topk_ids), _p(topk_w), _p(z), _p(gap), _p(ws), ws.numel(),
                                        _s(stream)))


def route_capped(shape, x, w_router, bias, w_down, promoted, k_hi, topk_ids, topk_w, z, gap, ws, stream=None):
    """moe_route with the moe_k_hi cap: promoted experts past the first k_hi of a token get weight 0."""
    check("moe_route_capped",
          load().moe_route_capped(shape, x.shape[0], _p(x), _p(w_router), _p(bias), _p(w_down), _p(promoted),
                                  int(k_hi), _p(topk_ids), _p(topk_w), _p(z), _p(gap), _p(ws), ws.numel(),
                                  _s(stream)))


def permute(shape, topk_ids, offsets, sorted_pair, pair_pos, active, ws, stream=None):
    check("moe_permute", load().moe_permute(shape, topk_ids.shape[0], _p(topk_ids), _p(offsets),
                                            _p(sorted_pair), _p(pair_pos), _p(active), _p(ws),
                                            ws.numel(), _s(stream)))


def grouped_gemm(shape, op, P, offsets, sorted_pair, A, w_packed, w_scale, w3_packed, w3_scale,
                 pair_weight, C, ws, stream=None, a_dtype=None):
    """mxfp4_grouped_gemm; a_rows is A's row count.  a_dtype defaults to the
    dtype of A (bf16 bits or fp32); MOE_DT_BF16X2 marks A as H planes."""
    if a_dtype is None:
        a_dtype = MOE_DT_BF16 if A.dtype in (torch.bfloat16, torch.int16, torch.uint16) else MOE_DT_F32
    check("mxfp4_grouped_gemm",
          load().mxfp4_grouped_gemm(shape, op, P, _p(offsets), _p(sorted_pair), _p(A), A.shape[0], a_dtype,
                                    _p(w_packed), _p(w_scale), _p(w3_packed), _p(w3_scale),
                                    _p(pair_weight), _p(C), _p(ws), ws.numel(), _s(stream)))


def expert_bank(fmt, n_experts, tensors, op):
    """moe_expert_bank for `op` from {w1,w3,w2}_{packed,scale[,bias]} tensors (stacked over the bank)."""
    mats = ("w1", "w3") if op == MOE_OP_GATEUP_SITU else ("w2", None)
    b = _lib.MoeExpertBank()
    b.format, b.n_experts = int(fmt), int(n_experts)
    if n_experts == 0:
        return b
    aff = fmt == _lib.MOE_WF_AFFINE2
    b.packed, b.scale = _p(tensors[mats[0] + "_packed"]), _p(tensors[mats[0] + "_scale"])
    b.bias = _p(tensors[mats[0] + "_bias"]) if aff else None
    if mats[1]:
        b.packed3, b.scale3 = _p(tensors[mats[1] + "_packed"]), _p(tensors[mats[1] + "_scale"])
        b.bias3 = _p(tensors[mats[1] + "_bias"]) if aff else None
    return b


def grouped_gemm_two_bank(shape, op, P, offsets, sorted_pair, A, bank_a, bank_b, pair_weight, C, ws, stream=None):
    """moe_grouped_gemm_two_bank; bank_a / bank_b are moe_expert_bank structs (see expert_bank)."""
    a_dtype = MOE_DT_BF16 if A.dtype in (torch.bfloat16, torch.int16, torch.uint16) else MOE_DT_F32
    check("moe_grouped_gemm_two_bank",
          load().moe_grouped_gemm_two_bank(shape, op, P, _p(offsets), _p(sorted_pair), _p(A), A.shape[0], a_dtype,
                                           bank_a, bank_b, _p(pair_weight), _p(C), _p(ws), ws.numel(), _s(stream)))


def combine_norm_up(shape, T, Y, pair_pos, topk_w, gamma, w_up, out, accumulate, ws, stream=None):
    check("moe_combine_norm_up",
          load().moe_combine_norm_up(shape, T, _p(Y), _p(pair_pos), _p(topk_w), _p(gamma), _p(w_up),
                                     _p(out), int(accumulate), _p(ws), ws.numel(), _s(stream)))


def shared_ffn(shape, x, w_gate, w_up, w_down, out, accumulate, ws, stream=None):
    check("shared_expert_ffn",
          load().shared_expert_ffn(shape, x.shape[0], _p(x), _p(w_gate), _p(w_up), _p(w_down), _p(out),
                                   int(accumulate), _p(ws), ws.numel(), _s(stream)))


def reap_saliency(shape, P, offsets, Y, pair_weight, sorted_pair, sal_sum, counts, accumulate, ws, stream=None):
    """REAP saliency numerator (float64 [E]) and token counts (int64 [E]), see moe_reap_saliency."""
    check("moe_reap_saliency",
          load().moe_reap_saliency(shape, int(P), _p(offsets), _p(Y), _p(pair_weight), _p(sorted_pair),
                                   _p(sal_sum), _p(counts), int(accumulate), _p(ws),
                                   0 if ws is None else ws.numel(), _s(stream)))


def combine_norm_up_reap(shape, T, Y, pair_pos, topk_w, gamma, w_up, out, accumulate, offsets, sal_sum, counts,
                         reap_accumulate, ws, stream=None):
    """moe_combine_norm_up plus the REAP saliency sums of the batch, see moe_combine_norm_up_reap."""
    check("moe_combine_norm_up_reap",
          load().moe_combine_norm_up_reap(shape, T, _p(Y), _p(pair_pos), _p(topk_w), _p(gamma), _p(w_up),
                                          _p(out), int(accumulate), _p(offsets), _p(sal_sum), _p(counts),
                                          int(reap_accumulate), _p(ws), ws.numel(), _s(stream)))


WEIGHT_KEYS = ("w_router", "bias", "w_down", "w_up", "gamma", "sh_gate", "sh_up", "sh_down",
               "w1_packed", "w1_scale", "w3_packed", "w3_scale", "w2_packed", "w2_scale")


# token counts up to which the dense products stream their weights (the
# decode-sized path); the latent projection then runs on the side stream
LATENT_SIDE_MAX_T = 64


_SIDE_STREAMS: dict = {}


def _side_stream(device: torch.device) -> torch.cuda.Stream:
    key = device.index if device.index is not None else torch.cuda.current_device()
    if key not in _SIDE_STREAMS:
        _SIDE_STREAMS[key] = torch.cuda.Stream(device=device)
    return _SIDE_STREAMS[key]


class LatentMoE:
    """One Stable LatentMoE layer on the GPU: weights resident, buffers per token count.

    forward(x) enqueues on a side stream, at decode sizes, the latent
    projection (moe_route without a router, writes z) and then the shared
    experts (shared_expert_ffn, writes out); on the caller's stream: moe_route
    (router and top-k, plus z at prefill sizes), moe_permute, then, once z is
    there, mxfp4_grouped_gemm (gate/up + SiTU-GLU), mxfp4_grouped_gemm (down)
    and, once the shared experts are done, moe_combine_norm_up (adds the
    routed part to out).  The side stream's work depends only on x, so it
    overlaps the latency-bound routing steps; the two output parts are added
    once, so the result is the same as running the calls in sequence.

    z runs on the side stream only at decode-sized token counts (T <= 64);
    latent_on_side=False keeps it on the caller's stream always.
    late_shared_join=False joins the whole side stream before the expert
    GEMMs instead (at decode sizes that puts the shared experts on the path to
    the expert GEMMs; at prefill sizes the two joins measure the same).
    overlap_shared=False runs everything on the caller's stream.

    h_planes: where the expert GEMMs take the tiled path (T k >= 8 E, single
    bank, operand mode BF16X2 or BF16) the gate/up call writes H as bf16
    hi + lo planes (buffer "H", int16 bits [T k, 2 I]) and the down call
    reads them, with no split pass in between; Y and the output are bitwise
    those of the fp32 H.  h_planes=False keeps H in fp32 always.
    """

    def __init__(self, shape: MoeShape, weights: dict, device="cuda", overlap_shared: bool = True,
                 latent_on_side: bool = True, late_shared_join: bool = True, bank_b: dict | None = None,
                 h_planes: bool = True):
        missing = [k for k in WEIGHT_KEYS if k not in weights]
        if missing:
            raise ValueError(f"missing weights: {missing}")
        self.shape = shape
        self.w = weights
        # two-bank layer: the w1/w3/w2 tensors hold bank A (the first n_a experts,
        # MXFP4) and bank_b = {"format": MOE_WF_*, "n_experts": n_b, tensors...}
        # holds the rest; the expert GEMMs then run moe_grouped_gemm_two_bank
        self.bank_b = bank_b
        if bank_b is not None:
            n_b = int(bank_b["n_experts"])
            n_a = shape.n_experts - n_b
            self._banks = {op: (expert_bank(_lib.MOE_WF_MXFP4, n_a, weights, op),
                                expert_bank(bank_b["format"], n_b, bank_b, op))
                           for op in (MOE_OP_GATEUP_SITU, MOE_OP_DOWN)}
        self.device = torch.device(device)
        self._bufs: dict = {}
        self.overlap_shared = overlap_shared
        # at decode sizes the latent projection z joins the shared experts on
        # the side stream, so the main stream's routing is only the router and
        # the top-k; at prefill sizes z stays on the main stream, where it runs
        # beside the shared experts instead of after them
        self.latent_on_side = latent_on_side and overlap_shared
        # late join: z runs first on the side stream and the expert GEMMs wait
        # only for it; the shared experts then overlap the expert GEMMs and are
        # joined before moe_combine_norm_up, which adds onto their output
        self.late_shared_join = late_shared_join and overlap_shared
        # default-priority side stream for the shared experts, one per device for
        # every layer object: the runtime maps streams onto a few hardware
        # queues, and with a stream per layer the side streams came to share the
        # caller's queue, where the overlap was lost (decode 0.756 ms a step with
        # the first layers' streams, 0.771 later)
        self.side = _side_stream(self.device) if overlap_shared else None
        self.h_planes = h_planes

    def planes_for(self, T: int) -> bool:
        """Whether H travels as bf16 planes at T tokens (see h_planes)."""
        s = self.shape
        return (self.h_planes and self.bank_b is None and s.operand_mode in (_lib.MOE_OPND_BF16X2, _lib.MOE_OPND_BF16)
                and T * s.top_k >= 8 * s.n_experts)

    def buffers(self, T: int) -> dict:
        if T in self._bufs:
            return self._bufs[T]
        s, dev = self.shape, self.device
        P = T * s.top_k
        gfn = _lib.MOE_FN_GROUPED_GEMM_TWO_BANK if self.bank_b is not None else MOE_FN_GROUPED_GEMM
        ws = max(workspace_bytes(s, fn, P if fn == gfn else T)
                 for fn in (MOE_FN_ROUTE, MOE_FN_PERMUTE, gfn, MOE_FN_COMBINE_NORM_UP))
        ws_sh = max(16, workspace_bytes(s, MOE_FN_SHARED_FFN, T), workspace_bytes(s, MOE_FN_ROUTE, T))
        i32, f32 = torch.int32, torch.float32
        b = {
            "topk_ids": torch.empty((T, s.top_k), dtype=i32, device=dev),
            "topk_w": torch.empty((T, s.top_k), dtype=f32, device=dev),
            "z": torch.empty((T, s.latent), dtype=f32, device=dev),
            "gap": torch.empty((T,), dtype=f32, device=dev),
            "offsets": torch.empty((s.n_experts + 1,), dtype=i32, device=dev),
            "sorted_pair": torch.empty((P,), dtype=i32, device=dev),
            "pair_pos": torch.empty((P,), dtype=i32, device=dev),
            "active": torch.empty((s.n_experts + 1,), dtype=i32, device=dev),
            "H": (torch.empty((P, 2 * s.inter), dtype=torch.int16, device=dev) if self.planes_for(T)
                  else torch.empty((P, s.inter), dtype=f32, device=dev)),
            "Y": torch.empty((P, s.latent), dtype=f32, device=dev),
            "out": torch.empty((T, s.hidden), dtype=f32, device=dev),
            "ws": torch.empty((ws,), dtype=torch.uint8, device=dev),
            "ws_shared": torch.empty((ws_sh,), dtype=torch.uint8, device=dev),
        }
        self._bufs[T] = b
        return b

    def forward(self, x: torch.Tensor, stream=None, marks: list | None = None, mark_names=None) -> dict:
        """Enqueue the layer.  With `marks` given, timing events are recorded
        around every call (or the calls named in `mark_names`) on the stream
        it runs on, appended as (name, start_event, end_event)."""
        s, w = self.shape, self.w
        T = x.shape[0]
        P = T * s.top_k
        b = self.buffers(T)
        ws = b["ws"]
        st = torch.cuda.current_stream() if stream is None else stream
        side = self.side if self.overlap_shared else st

        def call(name, strm, fn):
            if marks is None or (mark_names is not None and name not in mark_names):
                fn()
                return
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(strm)
            fn()
            e1.record(strm)
            marks.append((name, e0, e1))

        shared = s.n_shared * s.shared_inter > 0
        lat_side = self.latent_on_side and T <= LATENT_SIDE_MAX_T
        late = self.late_shared_join
        z_done = None
        if shared and side is not st:
            # side stream: the shared experts, during the latency-bound routing steps
            side.wait_stream(st)
            x.record_stream(side)
            latent = lambda: call("moe_route_latent", side,  # noqa: E731
                                  lambda: route(s, x, None, None, w["w_down"], None, None, b["z"], None,
                                                b["ws_shared"], side))
            if lat_side and late:
                latent()
                z_done = torch.cuda.Event()
                z_done.record(side)
            call("shared_expert_ffn", side,
                 lambda: shared_ffn(s, x, w["sh_gate"], w["sh_up"], w["sh_down"], b["out"], 0, b["ws_shared"],
                                    side))
            if lat_side and not late:
                latent()
            side_done = torch.cuda.Event()
            side_done.record(side)
        elif shared:
            call("shared_expert_ffn", st,
                 lambda: shared_ffn(s, x, w["sh_gate"], w["sh_up"], w["sh_down"], b["out"], 0, b["ws_shared"],
                                    st))
        z_main = not (shared and side is not st and lat_side)
        call("moe_route", st, lambda: route(s, x, w["w_router"], w["bias"], w["w_down"] if z_main else None,
                                            b["topk_ids"], b["topk_w"], b["z"] if z_main else None, b["gap"],
                                            ws, st))
        call("moe_permute", st, lambda: permute(s, b["topk_ids"], b["offsets"], b["sorted_pair"], b["pair_pos"],
                                                b["active"], ws, st))
        if shared and side is not st:
            if not late:
                # the expert GEMMs stream weights at full bandwidth on their own
                st.wait_event(side_done)
            elif z_done is not None:
                st.wait_event(z_done)
        if self.bank_b is not None:
            ga, gb = self._banks[MOE_OP_GATEUP_SITU]
            da, db = self._banks[MOE_OP_DOWN]
            call("grouped_gemm_gateup", st,
                 lambda: grouped_gemm_two_bank(s, MOE_OP_GATEUP_SITU, P, b["offsets"], b["sorted_pair"], b["z"], ga,
                                               gb, None, b["H"], ws, st))
            call("grouped_gemm_down", st,
                 lambda: grouped_gemm_two_bank(s, MOE_OP_DOWN, P, b["offsets"], b["sorted_pair"], b["H"], da, db,
                                               None, b["Y"], ws, st))
        else:
            planes = self.planes_for(T)
            call("grouped_gemm_gateup", st,
                 lambda: grouped_gemm(s, MOE_OP_GATEUP_SITU_BF16X2 if planes else MOE_OP_GATEUP_SITU, P,
                                      b["offsets"], b["sorted_pair"], b["z"], w["w1_packed"], w["w1_scale"],
                                      w["w3_packed"], w["w3_scale"], None, b["H"], ws, st))
            call("grouped_gemm_down", st,
                 lambda: grouped_gemm(s, MOE_OP_DOWN, P, b["offsets"], b["sorted_pair"], b["H"], w["w2_packed"],
                                      w["w2_scale"], None, None, None, b["Y"], ws, st,
                                      a_dtype=MOE_DT_BF16X2 if planes else None))
        if shared and side is not st and late:
            st.wait_event(side_done)
        call("moe_combine_norm_up", st,
             lambda: combine_norm_up(s, T, b["Y"], b["pair_pos"], b["topk_w"], w["gamma"], w["w_up"], b["out"],
                                     1 if shared else 0, ws, st))
        return b

"""The fused ShortConv K/V step as a differentiable torch op, for training.

``shortconv_kv(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps, k_init=None,
v_init=None)`` returns ``(y_k, y_v, k_state, v_state)``:

* ``y_k``, ``y_v``  [T, H, D]: the step's output rows (the rows the prefill writes into the cache,
  here written to fresh tensors in token order);
* ``k_state``, ``v_state``  [N, W-1, H, D]: each sequence's new conv state (its last W-1 raw rows),
  for the next chunk of a chunked sequence; None when W == 1.

``k_init``, ``v_init`` [N, W-1, H, D] are the sequences' initial windows (the previous chunk's new
state), or None for fresh sequences (zeros). Gradients flow to k, v, the taps, the gammas and the
initial windows, through the library's backward (``shortconv_kv_backward``); a loss on the new
states flows back too. Both directions run in the HIP library; this module only allocates
tensors and calls the C ABI through the binding.
"""
from typing import Optional

import torch

from . import _binding


class _ShortConvKV(torch.autograd.Function):
    @staticmethod
    def forward(ctx, k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps, k_init, v_init):
        W, H, D = k_taps.shape
        T, N = k.shape[0], cu_seqlens.shape[0] - 1
        dev = k.device
        y_k = torch.empty((T, H, D), dtype=k.dtype, device=dev)
        y_v = torch.empty_like(y_k)
        slots = torch.arange(T, dtype=torch.int64, device=dev)
        sidx = torch.arange(N, dtype=torch.int32, device=dev)
        fresh = k_init is None
        if W > 1:
            shape = (N, W - 1, H, D)
            k_pool = torch.zeros(shape, dtype=k.dtype, device=dev) if fresh else k_init.clone()
            v_pool = torch.zeros(shape, dtype=k.dtype, device=dev) if fresh else v_init.clone()
        else:
            k_pool = v_pool = None
        hinit = torch.full((N,), 0 if fresh else 1, dtype=torch.uint8, device=dev)
        _binding.shortconv_kv_prefill(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps,
                                      k_pool, v_pool, sidx, hinit, slots, y_k, y_v)
        ctx.save_for_backward(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, k_init, v_init)
        ctx.eps = eps
        ctx.fresh = fresh
        return y_k, y_v, k_pool, v_pool

    @staticmethod
    def backward(ctx, dy_k, dy_v, ds_k, ds_v):
        k, v, cu, k_taps, v_taps, k_gamma, v_gamma, k_init, v_init = ctx.saved_tensors
        W, H, D = k_taps.shape
        T, N = k.shape[0], cu.shape[0] - 1
        dev = k.device
        dy_k = torch.zeros_like(k) if dy_k is None else dy_k.contiguous()
        dy_v = torch.zeros_like(v) if dy_v is None else dy_v.contiguous()
        sidx = torch.arange(N, dtype=torch.int32, device=dev)
        hinit = torch.full((N,), 0 if ctx.fresh else 1, dtype=torch.uint8, device=dev)
        dk, dv = torch.empty_like(k), torch.empty_like(v)
        grads = [torch.empty_like(k_taps), torch.empty_like(v_taps), torch.empty_like(k_gamma),
                 torch.empty_like(v_gamma)]
        want_init = W > 1 and not ctx.fresh and (ctx.needs_input_grad[8] or
                                                 ctx.needs_input_grad[9])
        d_init = ((torch.empty((N, W - 1, H, D), dtype=k.dtype, device=dev),
                   torch.empty((N, W - 1, H, D), dtype=k.dtype, device=dev))
                  if want_init else (None, None))
        have_ds = W > 1 and (ds_k is not None or ds_v is not None)
        if have_ds:
            zeros = torch.zeros((N, W - 1, H, D), dtype=k.dtype, device=dev)
            ds = (zeros if ds_k is None else ds_k.contiguous(),
                  zeros if ds_v is None else ds_v.contiguous())
        else:
            ds = (None, None)
        pool_k = k_init if not ctx.fresh else None
        pool_v = v_init if not ctx.fresh else None
        _binding.shortconv_kv_backward(k, v, cu, k_taps, v_taps, k_gamma, v_gamma, ctx.eps,
                                       pool_k, pool_v, sidx, hinit, dy_k, dy_v, dk, dv, *grads,
                                       dstate_out=ds, dstate_in=d_init)
        return (dk, dv, None, grads[0], grads[1], grads[2], grads[3], None, d_init[0],
                d_init[1])


def shortconv_kv(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps: float,
                 k_init: Optional[torch.Tensor] = None, v_init: Optional[torch.Tensor] = None):
    """Differentiable fused ShortConv K/V step (see the module docstring)."""
    if (k_init is None) != (v_init is None):
        raise ValueError("give both initial windows or neither")
    return _ShortConvKV.apply(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, float(eps),
                              k_init, v_init)

"""Multi-step continuous-batching driver: the scheduler's plan of each step
fed to the kernels ("LLM 推理引擎 Continuous Batching 与 PagedAttention",
§2.1-§2.2: at every step boundary the batch is recomposed, and one step
runs the prefill chunks and the decode rows together).

A thin wrapper over the native step executor (``pkv_server_*``): per step,
``pkv_server_plan`` runs the scheduler into pinned staging memory and
enqueues its copy to the device, the caller's ``rows_fn`` produces the new
tokens' rows (in a model: the layer's projections), and
``pkv_server_execute`` enqueues kv append, prefill and decode.
Marshalling only: the plan is computed by the native scheduler, the
attention by the kernels.
"""
from __future__ import annotations

import ctypes
import time

import numpy as np
import torch

from . import PkvError, Scheduler, _StepPlan, _check, _stream, load_library


class StepDriver:
    """Drives ``scheduler`` over the pools ``k_cache`` / ``v_cache``
    ([NB, Hkv, bs, D] fp16 on the GPU).  ``rows_fn(plan)`` returns device
    tensors (new_k, new_v [N, Hkv, D], q [N, Hq, D], fp16, contiguous) for
    the plan's new tokens in slot_mapping order: the prefill chunks' tokens,
    then one row per decode request; ``plan`` is a dict of host arrays (see
    ``step``)."""

    def __init__(self, scheduler: Scheduler, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 num_q_heads: int, scale: float, rows_fn, pad_block: int = 0,
                 stream=None):
        self._lib = load_library()
        NB, Hkv, bs, D = k_cache.shape
        self.kc, self.vc, self.rows_fn, self.stream = k_cache, v_cache, rows_fn, stream
        self.Hq, self.D = int(num_q_heads), D
        self._h = self._lib.pkv_server_create(
            scheduler._h, scheduler.bm._h, k_cache.data_ptr(), v_cache.data_ptr(),
            self.Hq, Hkv, D, NB, int(pad_block), scheduler.max_batch_size,
            scheduler.max_num_tokens, scheduler.max_seq_len, float(scale))
        if not self._h:
            raise PkvError("pkv_server_create: invalid arguments or out of memory")
        self.s = scheduler
        dev = k_cache.device
        self.out_pf = torch.empty((scheduler.max_num_tokens, self.Hq, D), dtype=torch.float32,
                                  device=dev)
        self.out_dec = torch.empty((scheduler.max_batch_size, self.Hq, D), dtype=torch.float32,
                                   device=dev)
        self.steps = 0
        self.plan_s = 0.0   # host seconds planning (scheduler, staging wait, copy enqueue)

    def close(self):
        if self._h:
            self._lib.pkv_server_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _arrays(self, p):
        P, Dn = p.num_prefill, p.num_decode
        ptrs = [ctypes.c_void_p() for _ in range(7)]
        _check(self._lib.pkv_server_plan_arrays(self._h, *[ctypes.byref(x) for x in ptrs]),
               "server_plan_arrays")

        def view(ptr, ctype, n):
            if n == 0 or not ptr.value:
                return np.zeros(0, np.int64 if ctype is ctypes.c_int64 else np.int32)
            return np.ctypeslib.as_array(ctypes.cast(ptr, ctypes.POINTER(ctype)), (n,)).copy()
        I64, I32 = ctypes.c_int64, ctypes.c_int32
        return dict(prefill_ids=view(ptrs[0], I64, P), cu_q_lens=view(ptrs[1], I32, P + 1),
                    prefill_lens=view(ptrs[2], I32, P), decode_ids=view(ptrs[3], I64, Dn),
                    decode_lens=view(ptrs[4], I32, Dn),
                    finished=view(ptrs[5], I64, p.num_finished),
                    preempted=view(ptrs[6], I64, p.num_preempted),
                    num_new_tokens=p.num_new_tokens)

    def step(self):
        """Plans and enqueues one step.  Returns (plan, prefill_out,
        decode_out): plan is a dict of host arrays (prefill_ids, cu_q_lens,
        prefill_lens, decode_ids, decode_lens, finished, preempted), the
        outputs are device tensors (views of the driver's buffers, valid
        until the next step) or None."""
        st = _stream(self.stream)
        p = _StepPlan()
        t0 = time.perf_counter()
        _check(self._lib.pkv_server_plan(self._h, ctypes.byref(p), st), "server_plan")
        self.plan_s += time.perf_counter() - t0
        self.steps += 1
        plan = self._arrays(p)
        if p.num_new_tokens == 0:
            return plan, None, None
        new_k, new_v, q = self.rows_fn(plan)
        _check(self._lib.pkv_server_execute(self._h, new_k.data_ptr(), new_v.data_ptr(),
                                            q.data_ptr(), self.out_pf.data_ptr(),
                                            self.out_dec.data_ptr(), st), "server_execute")
        out_pf = self.out_pf[:p.num_prefill_tokens] if p.num_prefill else None
        out_dec = self.out_dec[:p.num_decode] if p.num_decode else None
        return plan, out_pf, out_dec


__all__ = ["StepDriver", "PkvError"]

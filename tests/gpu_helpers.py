"""Shared helpers of the GPU parity tests (not collected: no test_ prefix)."""

import sys

import numpy as np
import torch

import oracle
import paged_kv_extend_amd as pkv
import workloads as wl

# parity bars: bf16 inputs max-abs 2e-2 and mean-abs 2e-3; fp32 inputs 1e-5
TOL = {"bf16": (2e-2, 2e-3), "fp32": (1e-5, 1e-5)}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(w, dev=None, sm_scale=None, logit_cap=None):
    dev = dev or wl.to_torch(w)
    pkv.extend_attention_fwd(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"],
                             dev["v_pool"], dev["qo_indptr"], dev["kv_indptr"], dev["kv_indices"],
                             sm_scale=w.sm_scale if sm_scale is None else sm_scale,
                             logit_cap=w.logit_cap if logit_cap is None else logit_cap)
    torch.cuda.synchronize()
    return dev


def out_f64(dev):
    return dev["o"].float().cpu().numpy().astype(np.float64)


def check(got, want, dtype, what=""):
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite outputs"
    err = np.abs(got - want)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    bar_max, bar_mean = TOL[dtype]
    say(f"  {what}: max-abs {mx:.3g} mean-abs {mean:.3g}")
    assert mx <= bar_max and mean <= bar_mean, f"{what}: max-abs {mx:.3g}, mean-abs {mean:.3g}"


"""Helpers for the GPU tests: run the HIP library through its Python binding.

Nothing here computes any step of the method; it moves seeded inputs to the
device, calls the C ABI, and brings results back."""
import numpy as np
import torch

import shared_token_tiled_amd as ts

DEV = "cuda"


def say(msg):
    """Name the case before each GPU step (flushed, so it survives a crash)."""
    print(msg, flush=True)


class Run:
    """A plan uploaded for one configuration, plus device weights and workspace."""

    def __init__(self, cfg, layers, k_max=None):
        self.cfg = cfg
        self.plan = ts.ts_plan_create(cfg["ndim"], cfg["grid"], cfg["tile"], cfg["stride"],
                                      blend=1 if cfg.get("blend", "ramp") == "hard" else 0)
        ts.ts_plan_upload(self.plan, cfg["head_dim"], cfg.get("rope_base", 10000.0))
        self.info = ts.ts_plan_get_info(self.plan)
        self.model = ts.model_desc(dict(cfg, n_layers=len(layers)))
        self.tens, self.structs = ts.device_layers(layers, cfg, DEV)
        need = max(ts.ts_workspace_size(self.model, self.plan, k) for k in range(-1, len(layers) + 1))
        self.ws = torch.empty(need, dtype=torch.uint8, device=DEV)

    def close(self):
        ts.ts_plan_destroy(self.plan)
        self.plan = None

    def stack(self, x, g, k):
        xi = torch.as_tensor(x, dtype=torch.float32).to(DEV).contiguous()
        gi = torch.as_tensor(g, dtype=torch.float32).to(DEV).contiguous()
        xo = torch.empty_like(xi)
        go = torch.empty(self.info.n_tiles, self.cfg["d"], dtype=torch.float32, device=DEV)
        if k == len(self.structs):
            ts.ts_tiled_forward(self.model, self.structs, self.plan, xi, gi, xo, go, self.ws)
        else:
            ts.ts_stack_forward(self.model, self.structs, self.plan, k, xi, gi, xo, go, self.ws)
        torch.cuda.synchronize()
        return xo.cpu().numpy().astype(np.float64), go.cpu().numpy().astype(np.float64)

    def merge_once(self, x, g, l):
        xi = torch.as_tensor(x, dtype=torch.float32).to(DEV).contiguous()
        gi = torch.as_tensor(g, dtype=torch.float32).to(DEV).contiguous()
        xo = torch.empty_like(xi)
        go = torch.empty(self.info.n_tiles, self.cfg["d"], dtype=torch.float32, device=DEV)
        ts.ts_merge_once_forward(self.model, self.structs, self.plan, l, xi, gi, xo, go, self.ws)
        torch.cuda.synchronize()
        return xo.cpu().numpy().astype(np.float64), go.cpu().numpy().astype(np.float64)

    def partial_share(self, x, g, k, share):
        """share: a set of "q", "o", "m"."""
        mask = (ts.TS_SHARE_Q if "q" in share else 0) | (ts.TS_SHARE_O if "o" in share else 0) | \
            (ts.TS_SHARE_M if "m" in share else 0)
        xi = torch.as_tensor(x, dtype=torch.float32).to(DEV).contiguous()
        gi = torch.as_tensor(g, dtype=torch.float32).to(DEV).contiguous()
        xo = torch.empty_like(xi)
        go = torch.empty(self.info.n_tiles, self.cfg["d"], dtype=torch.float32, device=DEV)
        ts.ts_partial_share_forward(self.model, self.structs, self.plan, k, mask, xi, gi, xo, go, self.ws)
        torch.cuda.synchronize()
        return xo.cpu().numpy().astype(np.float64), go.cpu().numpy().astype(np.float64)

    def shared_layer(self, x_all, layer_index=0):
        xa = torch.as_tensor(x_all, dtype=torch.float32).to(DEV).contiguous()
        ts.ts_shared_layer_forward(self.model, self.structs[layer_index], self.plan, xa, self.ws)
        torch.cuda.synchronize()
        return xa.cpu().numpy().astype(np.float64)


def max_rel(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / np.sqrt(np.mean(ref * ref)))


TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}

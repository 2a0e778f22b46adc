"""The scans and the gate projections as differentiable torch operations.

Each forward calls the library's forward entry point and keeps its saved
record (a uint8 tensor) for the backward; each backward calls the adjoint
entry point.  Nothing here computes: these classes only route tensors to the
C ABI.  Gradients come back in the dtypes of the inputs they belong to (BF16
streams in BF16, FP32 parameters in FP32, BF16 projection weights in BF16).
An output whose gradient is not needed passes a NULL cotangent (zero) to the
library.  The streams (x_sel, b; x, l^x, l^a) must be BF16, the library's
input format: a tensor of another dtype is refused rather than converted."""
import torch

from . import scan


def _need_bf16(**tensors):
    for name, t in tensors.items():
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be torch.bfloat16 (the scan's input format), got {t.dtype}")


class SamuScan(torch.autograd.Function):
    """SAMU mixer scan: (x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z0) ->
    (y [B, L, D/2, 2] BF16, z_final [B, D/2, 2] FP32)."""

    @staticmethod
    def forward(ctx, x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z0, K, G):
        _need_bf16(x_sel=x_sel, b=b)
        y, z_final, saved = scan.samu_scan_fwd(x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z0, K=K, G=G,
                                               y_dtype=torch.bfloat16)
        ctx.save_for_backward(x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, saved)
        ctx.K, ctx.G, ctx.has_z0 = K, G, z0 is not None
        ctx.set_materialize_grads(False)
        return y, z_final

    @staticmethod
    def backward(ctx, dy, dz_final):
        x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, saved = ctx.saved_tensors
        B, L, D = x_sel.shape
        if dy is None:
            dy = torch.zeros((B, L, D // 2, 2), dtype=torch.bfloat16, device=b.device)
        dy = dy.to(torch.bfloat16).contiguous()
        dzf = None if dz_final is None else dz_final.float().contiguous()
        g = scan.samu_scan_bwd(x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, saved, dy, dzf, K=ctx.K, G=ctx.G,
                               grad_dtype=torch.bfloat16, want_dz0=ctx.has_z0)
        return (g["dx_sel"], g["db"], g["dw_phi"], g["dw_r"], g["da_phi"], g["da_r"], g["dnu"],
                g["dtheta"], g["dz0"] if ctx.has_z0 else None, None, None)


class RglruScan(torch.autograd.Function):
    """RG-LRU scan: (x, lx, la, alpha, reset, h0) -> (y [B, L, D] BF16,
    h_final [B, D] FP32); `reset` (uint8 [B, L] or None) takes no
    gradient."""

    @staticmethod
    def forward(ctx, x, lx, la, alpha, reset, h0, K, G):
        _need_bf16(x=x, lx=lx, la=la)
        y, h_final, saved = scan.rglru_scan_fwd(x, lx, la, alpha, reset, h0, K=K, G=G, y_dtype=torch.bfloat16)
        ctx.save_for_backward(x, lx, la, alpha, reset, saved)
        ctx.K, ctx.G, ctx.has_h0 = K, G, h0 is not None
        ctx.set_materialize_grads(False)
        return y, h_final

    @staticmethod
    def backward(ctx, dy, dh_final):
        x, lx, la, alpha, reset, saved = ctx.saved_tensors
        if dy is None:
            dy = torch.zeros_like(x)
        dy = dy.to(torch.bfloat16).contiguous()
        dhf = None if dh_final is None else dh_final.float().contiguous()
        g = scan.rglru_scan_bwd(x, lx, la, alpha, reset, saved, dy, dhf, K=ctx.K, G=ctx.G,
                                grad_dtype=torch.bfloat16, want_dh0=ctx.has_h0)
        return (g["dx"], g["dlx"], g["dla"], g["dalpha"], None,
                g["dh0"] if ctx.has_h0 else None, None, None)


class RglruGateProj(torch.autograd.Function):
    """The two 16-block block-diagonal gate projections: (x, w_x, b_x, w_a,
    b_a) -> (l^x, l^a), BF16 [B, L, D]."""

    @staticmethod
    def forward(ctx, x, w_x, b_x, w_a, b_a):
        _need_bf16(x=x, w_x=w_x, w_a=w_a)
        lx, la = scan.rglru_gate_proj_fwd(x, w_x, b_x, w_a, b_a)
        ctx.save_for_backward(x, w_x, w_a)
        ctx.set_materialize_grads(False)
        return lx, la

    @staticmethod
    def backward(ctx, dlx, dla):
        x, w_x, w_a = ctx.saved_tensors
        ref = dlx if dlx is not None else dla
        if ref is None:
            return None, None, None, None, None
        dt = torch.float32 if ref.dtype == torch.float32 else torch.bfloat16  # the adjoint's cotangent types
        z = None
        if dlx is None or dla is None:
            z = torch.zeros(x.shape, dtype=dt, device=x.device)
        dlx = z if dlx is None else dlx.to(dt).contiguous()
        dla = z if dla is None else dla.to(dt).contiguous()
        g = scan.rglru_gate_proj_bwd(x, w_x, w_a, dlx, dla, torch.zeros(x.shape, dtype=dt, device=x.device))
        return (g["dx"].to(x.dtype), g["dw_x"].to(w_x.dtype), g["db_x"], g["dw_a"].to(w_a.dtype), g["db_a"])


def samu_scan(x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z0=None, *, K=32, G=0):
    return SamuScan.apply(x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z0, K, G)


def rglru_scan(x, lx, la, alpha, reset=None, h0=None, *, K=16, G=0):
    return RglruScan.apply(x, lx, la, alpha, reset, h0, K, G)


def rglru_gate_proj(x, w_x, b_x, w_a, b_a):
    return RglruGateProj.apply(x, w_x, b_x, w_a, b_a)


class RglruLayer(torch.autograd.Function):
    """Input to output of the RG-LRU layer as one differentiable operation:
    the two gate projections, then the scan.  x feeds both, so its gradient
    has two terms: the backward runs the scan adjoint with FP32 cotangents,
    accumulates the projection adjoint into that FP32 dx in place (the
    library's dx_in accumulate), and rounds the sum to BF16 once."""

    @staticmethod
    def forward(ctx, x, w_x, b_x, w_a, b_a, alpha, reset, h0, K, G):
        _need_bf16(x=x, w_x=w_x, w_a=w_a)
        lx, la = scan.rglru_gate_proj_fwd(x, w_x, b_x, w_a, b_a)
        y, h_final, saved = scan.rglru_scan_fwd(x, lx, la, alpha, reset, h0, K=K, G=G, y_dtype=torch.bfloat16)
        ctx.save_for_backward(x, w_x, w_a, lx, la, alpha, reset, saved)
        ctx.K, ctx.G, ctx.has_h0 = K, G, h0 is not None
        ctx.set_materialize_grads(False)
        return y, h_final

    @staticmethod
    def backward(ctx, dy, dh_final):
        x, w_x, w_a, lx, la, alpha, reset, saved = ctx.saved_tensors
        if dy is None:
            dy = torch.zeros_like(x)
        dy = dy.to(torch.bfloat16).contiguous()
        dhf = None if dh_final is None else dh_final.float().contiguous()
        g = scan.rglru_scan_bwd(x, lx, la, alpha, reset, saved, dy, dhf, K=ctx.K, G=ctx.G,
                                grad_dtype=torch.float32, want_dh0=ctx.has_h0)
        p = scan.rglru_gate_proj_bwd(x, w_x, w_a, g["dlx"], g["dla"], g["dx"], dx_out=g["dx"])
        return (p["dx"].to(torch.bfloat16), p["dw_x"].to(w_x.dtype), p["db_x"], p["dw_a"].to(w_a.dtype),
                p["db_a"], g["dalpha"], None, g["dh0"] if ctx.has_h0 else None, None, None)


def rglru_layer(x, w_x, b_x, w_a, b_a, alpha, reset=None, h0=None, *, K=16, G=0):
    """Input to output of the RG-LRU layer: gate projections, then the scan
    (one autograd node; x's gradient is rounded to BF16 once)."""
    return RglruLayer.apply(x, w_x, b_x, w_a, b_a, alpha, reset, h0, K, G)

"""Walk-resident serial draft head for MI355X (gfx950).

Python face of libwts.so ("Weights That Stay", arXiv 2611.00506): torch
tensors supply device memory and streams; every step of the walk runs in the
library's HIP kernels.  See include/wts.h for the C ABI.
"""
import ctypes

from . import _abi
from ._abi import WtsError, EXEC, HEAD, WTYPE  # noqa: F401

__all__ = ["Head", "WtsError", "check_log_ratio", "roofline"]


def check_log_ratio(device=0):
    """Mismatches between the kernels' log-argument quotient and the IEEE
    division over every reduced argument (wts_check_log_ratio); 0 expected."""
    n = ctypes.c_int64(-1)
    _check(_abi.lib().wts_check_log_ratio(int(device), ctypes.byref(n)), "wts_check_log_ratio")
    return n.value


def roofline(device=0):
    """Measured roofline denominators on `device` (wts_roofline): LDS read and
    MFMA issue rates, shader clock, HBM and memory-side-cache stream rates, the
    cross-workgroup selection round of four exchange designs, one-way signal
    hops and VALU issue cycles.  Returns a dict."""
    r = _abi.RooflineResult()
    _check(_abi.lib().wts_roofline(int(device), ctypes.byref(r)), "wts_roofline")
    return r.as_dict()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(code, what):
    if code != _abi.WTS_OK:
        raise WtsError(code, what)


class Head:
    """One serial draft head on one GPU.

    W: int8 [V, 256] (with w_scale float32 [V]) or bf16 [V, 256]; E float32
    [V, 256]; recurrent heads also take A bf16 [256, 256] and c float32 [256].
    All tensors live on the same CUDA (HIP) device and are borrowed until
    close().  grid: workgroups of the persistent walk (0: one per compute
    unit).  exchange: "auto" (the first selection level inside one XCD when
    the create-time dispatch check passes) or "device" (device scope).
    """

    def __init__(self, W, E, *, w_scale=None, A=None, c=None, head="markov", max_batch=16,
                 max_steps=64, resident_tiles=-1, lds_tiles=-1, cooperative=False, watchdog_us=0, grid=0,
                 exchange="auto"):
        import torch
        self._torch = torch
        wtype = "int8" if W.dtype == torch.int8 else "bf16"
        if wtype == "bf16" and W.dtype != torch.bfloat16:
            raise TypeError("W must be int8 or bfloat16")
        for t in (W, E, w_scale, A, c):
            if t is not None and not (t.is_cuda and t.is_contiguous()):
                raise ValueError("tensors must be contiguous and on the GPU")
        self._keep = (W, E, w_scale, A, c)
        self.V, self.r = W.shape
        self.head, self.wtype = head, wtype
        self.device = W.device
        p = _abi.CreateParams(V=self.V, r=self.r, head=HEAD[head], wtype=WTYPE[wtype], W=_ptr(W),
                              w_scale=_ptr(w_scale), E=_ptr(E), A=_ptr(A), c=_ptr(c), max_batch=max_batch,
                              max_steps=max_steps, resident_tiles=resident_tiles, lds_tiles=lds_tiles,
                              device=W.device.index or 0, cooperative=int(bool(cooperative)),
                              watchdog_us=watchdog_us, grid=grid,
                              exchange={"auto": 0, "device": 1}[exchange])
        h = ctypes.c_void_p()
        _check(_abi.lib().wts_create(ctypes.byref(p), ctypes.byref(h)), "wts_create")
        self._h = h

    def plan(self, B=1, exec="resident", temperature=0):
        p = _abi.Plan()
        _check(_abi.lib().wts_get_plan(self._h, B, EXEC[exec], temperature, ctypes.byref(p)), "wts_get_plan")
        return p.as_dict()

    def walk(self, base, x0, *, h0=None, temperature=0, seed=0, step_offset=0, logits=False,
             state=False, lse=False, exec="resident", fixed_latent=False, stream=None, out=None,
             trace=False, noalloc=False, stress=False, winners=False):
        """Enqueue one walk.  base: bf16 [B, gamma, V]; x0: int32 [B].

        Returns a dict of output tensors (tokens int32 [B, gamma]; logits bf16
        [B, gamma, V], state float32 [B, 256], lse float32 [B, gamma] (log
        normaliser of each step's logits) and trace int64 [gamma, grid, 4]
        when asked for).  fixed_latent runs the fixed-latent probe (every step
        uses the latent of step 0).  Pass `out` (a dict from an earlier call)
        to reuse its buffers.  noalloc=True runs the walk through
        wts_walk_noalloc (scratch in the library's fixed per-GPU array).
        stress delays workgroups at random before each selection; winners
        returns the key each workgroup observed (uint64 as int64 [gamma, B,
        grid]); both for testing the selection.
        """
        torch = self._torch
        B, gamma, V = base.shape
        if out is None:
            out = {"tokens": torch.empty((B, gamma), dtype=torch.int32, device=self.device)}
            if logits:
                out["logits"] = torch.empty((B, gamma, V), dtype=torch.bfloat16, device=self.device)
            if state:
                out["state"] = torch.empty((B, self.r), dtype=torch.float32, device=self.device)
            if trace:
                out["trace"] = torch.zeros((gamma, self.plan(B)["grid"], 4), dtype=torch.int64,
                                           device=self.device)
            if lse:
                out["lse"] = torch.empty((B, gamma), dtype=torch.float32, device=self.device)
            if winners:
                out["winners"] = torch.zeros((gamma, B, self.plan(B)["grid"]), dtype=torch.int64,
                                             device=self.device)
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        p = _abi.WalkParams(B=B, gamma=gamma, step_offset=step_offset, temperature=temperature,
                            seed=seed, base=_ptr(base), x0=_ptr(x0), h0=_ptr(h0),
                            tokens_out=_ptr(out["tokens"]), logits_out=_ptr(out.get("logits")),
                            state_out=_ptr(out.get("state")), exec=EXEC[exec],
                            flags=(_abi.WALK_FIXED_LATENT if fixed_latent else 0) | (_abi.WALK_STRESS if stress else 0),
                            stream=ctypes.c_void_p(s.cuda_stream), trace_out=_ptr(out.get("trace")),
                            lse_out=_ptr(out.get("lse")), winners_out=_ptr(out.get("winners")))
        if noalloc:
            _check(_abi.lib().wts_walk_noalloc(self._h, ctypes.byref(p)), "wts_walk_noalloc")
        else:
            _check(_abi.lib().wts_walk(self._h, ctypes.byref(p)), "wts_walk")
        return out

    def error(self, clear=True):
        """Synchronize and return the device-latched status name (WTS_OK if none)."""
        return _abi.STATUS_NAMES[_abi.lib().wts_get_error(self._h, 1 if clear else 0)]

    def close(self):
        if getattr(self, "_h", None):
            _abi.lib().wts_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

"""Shared test helpers: run the HIP path through the C ABI and the oracle on the same inputs."""
import numpy as np
import torch

from hybrid_linear_attention_prefill_amd import synth

TOL = 2e-3  # relative L2 bound on outputs and final state against the float64 oracle


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def bits(t):
    """Raw bits of a tensor as an integer numpy array (bitwise comparisons)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy()
    return t.numpy()


def same_bits(a, b):
    return a.shape == b.shape and np.array_equal(bits(a), bits(b))


def desc_kwargs(desc):
    return dict(n_k_heads=desc.n_k_heads, n_v_heads=desc.n_v_heads, d_k=desc.d_k, d_v=desc.d_v,
                scale=float(desc.scale), l2_eps=float(desc.l2_eps), conv_silu=bool(desc.conv_silu))


def oracle(desc, inp, S0=None, window=None, heads=None, want_o=True):
    """Float64 oracle on the exact (cast) inputs.  Returns (o, S, window_out)."""
    from oracle import c_oracle
    x = synth.f64(inp["x"])
    T, C = x.shape
    if S0 is None:
        S0 = np.zeros((desc.n_v_heads, desc.d_k, desc.d_v))
    conv_w = synth.f64(inp["conv_w"]) if desc.conv_width > 0 else None
    if desc.conv_width > 0 and window is None:
        window = np.zeros((desc.conv_width - 1, C))
    return c_oracle.gdn_layer(x, conv_w, window, synth.f64(inp["g"]), synth.f64(inp["beta"]),
                              S0, heads=heads, want_o=want_o, **desc_kwargs(desc))


def to_dev(inp, device="cuda"):
    return {k: v.to(device) for k, v in inp.items()}


def new_state(b, desc, zero=True):
    s = b.State(desc)
    if zero:
        b.gdn_state_init(desc, s)
    return s


def run_fork(b, desc, dinp, state_in, rows=None, out_state=None, ws=None):
    """FORK from state_in over rows [r0, r1) of the device inputs; returns (o, out_state)."""
    r0, r1 = rows if rows is not None else (0, dinp["x"].shape[0])
    T = r1 - r0
    o = torch.empty((T, desc.n_v_heads, desc.d_v), dtype=desc.out_torch, device="cuda")
    out_state = out_state or b.State(desc)
    ws = ws if ws is not None else b.workspace(desc, T, 1)
    b.gdn_prefill_chunked(desc, dinp["x"][r0:r1], dinp.get("conv_w"), dinp["g"][r0:r1],
                          dinp["beta"][r0:r1], state_in, out_state, o, T, b.GDN_FORK, ws)
    return o, out_state

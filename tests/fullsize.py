"""Full-size parity runs: every state of a workload on the GPU, sampled states
checked against the oracle.

Two disjoint samples of states are followed:
  * forced: at the start of every window the GPU state of these states is
    overwritten with the oracle's own boundary state, so every window's
    outputs and closing boundary are compared strictly (the oracle never
    reads a GPU result);
  * free: never touched; compared strictly until a legitimate
    rounding-boundary flip makes the two trajectories part, then by a
    relative bound.
All other states run alongside in the same launches (the benchmark's launch
configuration: one decode launch per layer and token; either one window
close over all layers' states per window, or, with fused=True, the last
token of each window decoded and the window closed per layer in one
leapquant_decode_close launch).
"""
import numpy as np
import torch

import recurrent_state_quant_amd as lq
from oracle import leapquant_oracle as O
from tests import parity as P
from tests.gpu_run import to_np
from workloads import generators as G

DEV = "cuda"


def _gate(g):
    return O.GATE_GDN if g == "gdn" else O.GATE_KDA


def pick_states(cfg, n_forced, n_free, seed=1234):
    """Global state indices: the first and last state of every layer slab are
    always forced (edge workgroups), the rest drawn without replacement."""
    rng = np.random.default_rng(seed)
    nl = cfg.states_per_layer
    edges = []
    for l in range(cfg.layers):
        edges += [l * nl, l * nl + nl - 1]
    edges = sorted(set(edges))
    rest = np.setdiff1d(np.arange(cfg.n_states), edges)
    draw = rng.choice(rest, size=max(0, n_forced - len(edges)) + n_free, replace=False)
    forced = np.array(sorted(edges + draw[:max(0, n_forced - len(edges))].tolist()))
    free = np.array(sorted(draw[max(0, n_forced - len(edges)):].tolist()))
    return forced, free


def _gather_boundary(slab, idx):
    return {k: v.cpu().numpy() for k, v in slab.boundary(idx).items()}


def _inject(slab, idx, b):
    slab.load_boundary({k: np.ascontiguousarray(b[k]) for k in lq.LeapQuantState.BOUNDARY}, idx)


def _decode_window(slab, slabs, tok, w, p, nl, L, outs, fused, after_token=None):
    """One window of every layer: p - 1 decode steps and a fused last token
    per layer, or p decode steps and one close over the whole slab."""
    for j in range(p):
        t = w * p + j
        for l in range(L):
            sl = slice(l * nl, (l + 1) * nl)
            args = (tok["q"][t, sl], tok["k"][t, sl], tok["v"][t, sl], tok["beta"][t, sl],
                    tok["alpha"][t, sl], outs[l])
            if fused and j == p - 1:
                lq.leapquant_decode_close(slabs[l], j, *args)
            else:
                lq.leapquant_decode_step(slabs[l], j, *args)
            if after_token is not None:
                after_token(t, l)
    if not fused:
        lq.leapquant_window_close(slab, p)


def run(cfg, n_forced=8, n_free=8, steps=None, seed=None, log=None, checkpoint_every=0, fused=False):
    """Run the workload and compare.  With checkpoint_every > 0 (a multiple
    of p) the whole boundary state is snapshotted at every checkpoint (the
    prefix-cache shape), the state MSE of the free states against the exact
    fp64 recurrence is tracked for the GPU and for the oracle, and a resume
    from the middle snapshot is checked to reproduce the next snapshot bit
    for bit."""
    if log is None:
        def log(msg):
            print(msg, flush=True)
    steps = steps or cfg.steps
    T, p, nl, L = steps, cfg.p, cfg.states_per_layer, cfg.layers
    gate = _gate(cfg.gate)
    g = G.make_generator(cfg.seed if seed is None else seed, DEV)
    S0 = G.initial_state(cfg, cfg.n_states, g, DEV)
    tok = G.token_inputs(cfg, cfg.n_states, T, g, DEV)
    forced, free = pick_states(cfg, n_forced, n_free)
    both = np.concatenate([forced, free])
    both_t = torch.as_tensor(both, device=DEV)
    S0s = S0.index_select(0, both_t).cpu().numpy()
    toks = {k: v.index_select(1, both_t).cpu().numpy().astype(np.float64) for k, v in tok.items()}
    nf = len(forced)
    tok_f = {k: v[:, :nf] for k, v in toks.items()}
    tok_r = {k: v[:, nf:] for k, v in toks.items()}
    log(f"[fullsize {cfg.name}] oracle: {nf} forced + {len(free)} free states x {T} tokens"
        f" ({'fused last token' if fused else 'separate close'})")
    o_f, b_f = O.run_windowed(S0s[:nf], tok_f, p, cfg.r, gate)
    o_r, b_r = O.run_windowed(S0s[nf:], tok_r, p, cfg.r, gate) if len(free) else (None, None)

    # the benchmark's layout: one slab for all layers, decoded per layer
    # through views, quantized and window-closed in one launch
    slab = lq.LeapQuantState(cfg.n_states, p, cfg.r, cfg.gate, DEV)
    slabs = [slab.view(l * nl, nl) for l in range(L)]
    outs = [torch.empty((nl, cfg.dv), device=DEV) for _ in range(L)]
    lq.leapquant_quantize_state(slab, S0)
    # boundary 0 of the forced states must already agree bit for bit
    P.compare_boundary(_gather_boundary(slab, forced), b_f[0], S0s[:nf], cfg.r,
                       f"{cfg.name} boundary 0", exact=True)
    rec = torch.empty((T, len(both), cfg.dv), device=DEV)
    loc = [[(j, int(gi) - l * nl) for j, gi in enumerate(both) if int(gi) // nl == l] for l in range(L)]
    loc_t = [(torch.as_tensor([a for a, _ in lo], device=DEV, dtype=torch.long),
              torch.as_tensor([b for _, b in lo], device=DEV, dtype=torch.long)) for lo in loc]
    diverged = np.zeros(len(free), bool)
    stats = {"flips": 0, "codes": 0, "ties": 0, "max_half_dist": 0.0, "worst_free_rel": 0.0,
             "free_ties": 0, "free_parted": []}
    snaps, mse = {}, []
    if checkpoint_every:
        assert checkpoint_every % p == 0 and len(free)
        _, _, exact = O.sequential_exact(S0s[nf:], tok_r, gate, keep_every=checkpoint_every)
        deq = torch.empty((nl, cfg.dk, cfg.dv), device=DEV)
    def gather_outputs(t, l):
        dst, src = loc_t[l]
        if len(dst):
            rec[t].index_copy_(0, dst, outs[l].index_select(0, src))

    for w in range(T // p):
        _inject(slab, forced, b_f[w])
        _decode_window(slab, slabs, tok, w, p, nl, L, outs, fused, gather_outputs)
        ws = slice(w * p, (w + 1) * p)
        og = to_np(rec[ws])
        P.assert_close(og[:, :nf], o_f[ws], f"{cfg.name} window {w} forced outputs")
        _, recs, S_end, _ = O.window(b_f[w], tok_f, w * p, p, gate, cfg.r)
        s = P.compare_boundary(_gather_boundary(slab, forced), b_f[w + 1],
                               S_end.astype(np.float32), cfg.r, f"{cfg.name} boundary {w + 1}",
                               mag=P.rebuild_magnitude(b_f[w], recs))
        for k in ("flips", "codes", "ties"):
            stats[k] += s[k]
        stats["max_half_dist"] = max(stats["max_half_dist"], s["max_half_dist"])
        if len(free):
            ofr, orr = og[:, nf:], o_r[ws]
            strict = ~diverged
            if strict.any():
                P.assert_close(ofr[:, strict], orr[:, strict], f"{cfg.name} window {w} free outputs")
            if diverged.any():
                rel = np.linalg.norm(ofr[:, diverged] - orr[:, diverged]) / np.linalg.norm(orr[:, diverged])
                stats["worst_free_rel"] = max(stats["worst_free_rel"], float(rel))
                assert rel < 2e-2, f"{cfg.name} window {w}: diverged free states differ by {rel}"
            gb = _gather_boundary(slab, free)
            if strict.any():
                # free states still on the oracle's trajectory closed this
                # window from the oracle's boundary: checked strictly, so a
                # state parts only at a legitimate rounding flip or near tie
                sel = np.nonzero(strict)[0]
                _, rr, S_fr, _ = O.window(O.copy_boundary(b_r[w], sel), {k: v[:, sel] for k, v in tok_r.items()},
                                          w * p, p, gate, cfg.r)
                sf = P.compare_boundary({k: v[sel] for k, v in gb.items()}, O.copy_boundary(b_r[w + 1], sel),
                                        S_fr.astype(np.float32), cfg.r, f"{cfg.name} free boundary {w + 1}",
                                        mag=P.rebuild_magnitude(O.copy_boundary(b_r[w], sel), rr))
                stats["free_ties"] += sf["ties"]
                stats["max_half_dist"] = max(stats["max_half_dist"], sf["max_half_dist"])
            same = np.all(gb["codes"] == b_r[w + 1]["codes"], axis=(1, 2))
            if cfg.r:
                same &= np.all(gb["comp_idx"] == b_r[w + 1]["comp_idx"], axis=1)
            newly = strict & ~same
            if newly.any():
                stats["free_parted"].append((w + 1, int(newly.sum())))
            diverged |= ~same
        tt = (w + 1) * p
        if checkpoint_every and tt % checkpoint_every == 0:
            snaps[tt] = [sl_.snapshot() for sl_ in slabs]
            g_err, o_err = [], []
            for j, gi in enumerate(free):
                l, i = divmod(int(gi), nl)
                lq.leapquant_dequantize_state(slabs[l], deq)
                Bg = deq[i].double().cpu().numpy()
                g_err.append(((Bg - exact[tt][j]) ** 2).mean())
            o_err = O.state_mse(b_r[w + 1], exact[tt])
            mse.append((tt, float(np.mean(g_err)), float(np.mean(o_err))))
    torch.cuda.synchronize()
    if checkpoint_every:
        stats["mse"] = mse
        for tt, mg, mo in mse:
            assert mg <= 2.0 * mo + 1e-12 and mo <= 2.0 * mg + 1e-12, (tt, mg, mo)
        keys = sorted(snaps)
        mid = keys[len(keys) // 2 - 1] if len(keys) > 1 else None
        if mid is not None:
            nxt = mid + checkpoint_every
            rslab = lq.LeapQuantState(cfg.n_states, p, cfg.r, cfg.gate, DEV)
            res = [rslab.view(l * nl, nl) for l in range(L)]
            for l in range(L):
                res[l].load_boundary(snaps[mid][l])
            for w in range(mid // p, nxt // p):
                _decode_window(rslab, res, tok, w, p, nl, L, outs, fused)
            # forced states were overwritten by injection in the original run:
            # compare the states that ran untouched
            untouched = torch.ones(cfg.n_states, dtype=torch.bool)
            untouched[torch.as_tensor(forced)] = False
            for l in range(L):
                keep = untouched[l * nl:(l + 1) * nl].to(DEV)
                cur = res[l].boundary()
                for k in lq.LeapQuantState.BOUNDARY:
                    a_, b_ = cur[k][keep], snaps[nxt][l][k][keep]
                    assert torch.equal(a_, b_), f"resume from token {mid}: {k} differs at token {nxt}"
            stats["resume"] = (mid, nxt)
    stats["free_diverged"] = int(diverged.sum())
    log(f"[fullsize {cfg.name}] ok: {stats}")
    return stats

"""Oracle for the fused optimizer steps over a planned buffer (test
infrastructure; the product never imports it).

The pages hand a sharded DTensor's local parameters straight to PyTorch's
fused AdamW / SGD (veScale 深度技术分析, OpDispatcher: the fused AdamW/SGD
handler) and run 8-bit Adam on block-quantised optimizer states
(veScale-FSDP: Flexible and High-Performance FSDP at Scale, section 6.3).
They do not spell the update out; the plainest reading is the textbook one,
written here in fp32 with every operation rounded once and no fused
multiply-add:

AdamW (decoupled weight decay), per element, with c = 1/grad_scale:
    g   = grad * c
    m'  = beta1*m + (1-beta1)*g
    v'  = beta2*v + (1-beta2)*(g*g)
    den = sqrt(v') / sqrt(bc2) + eps
    p'  = p*(1 - lr*wd) - (lr/bc1) * (m' / den)
where bc1 = 1-beta1^t and bc2 = 1-beta2^t are given by the caller (fp32)
and the per-call constants (1-beta1, 1-beta2, 1-lr*wd, lr/bc1, sqrt(bc2),
1/grad_scale) are fp32 operations on the fp32 hyperparameters.

SGD with momentum (coupled weight decay, no dampening):
    g   = grad*c + wd*p
    b'  = mu*b + g
    d   = g + mu*b'  (nesterov)  or  b'
    p'  = p - lr*d

Only tensor elements of ranks [k0, k1) with mask[t] set are updated.  When
found_inf (u32[m]) has any non-zero entry the whole step is skipped, as the
sharded gradient scaler does after reducing found-inf across ranks
("PyTorch FSDP", native mixed precision section).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .plan import Item, fragments

F32 = np.float32


def adamw_constants(lr, beta1, beta2, eps, wd, bc1, bc2, grad_scale):
    lr, beta1, beta2, eps, wd, bc1, bc2, gs = (F32(v) for v in (lr, beta1, beta2, eps, wd, bc1,
                                                                bc2, grad_scale))
    one = F32(1)
    return dict(omb1=F32(one - beta1), omb2=F32(one - beta2), decay=F32(one - F32(lr * wd)),
                step=F32(lr / bc1), bc2s=F32(np.sqrt(bc2)), inv=F32(one / gs), beta1=beta1,
                beta2=beta2, eps=eps)


def adamw_elem(p, g, m, v, k):
    """The AdamW update on fp32 arrays (returns p', m', v')."""
    with np.errstate(all="ignore"):
        gg = (g * k["inv"]).astype(F32)
        m2 = (F32(k["beta1"] * m) + F32(k["omb1"] * gg)).astype(F32)
        v2 = (F32(k["beta2"] * v) + F32(k["omb2"] * F32(gg * gg))).astype(F32)
        den = (F32(np.sqrt(v2) / k["bc2s"]) + k["eps"]).astype(F32)
        upd = F32(m2 / den)
        p2 = (F32(p * k["decay"]) - F32(k["step"] * upd)).astype(F32)
    return p2, m2, v2


def _skip(found_inf) -> bool:
    return found_inf is not None and bool(np.any(np.asarray(found_inf) != 0))


def adamw_step(p, g, m, v, items: Sequence[Item], offsets, S, m_ranks, k0, k1, hp: dict,
               mask: Optional[Sequence[int]] = None, found_inf=None, inplace: bool = False):
    """AdamW over the buffer's tensor elements in ranks [k0, k1); padding and
    masked-off tensors untouched.  Returns new (p, m, v) (the inputs
    themselves when inplace)."""
    if not inplace:
        p, m, v = p.copy(), m.copy(), v.copy()
    if _skip(found_inf):
        return p, m, v
    k = adamw_constants(**hp)
    for tid, r, lo, hi in fragments(items, offsets, S, m_ranks):
        if not (k0 <= r < k1) or (mask is not None and not mask[tid]):
            continue
        p[lo:hi], m[lo:hi], v[lo:hi] = adamw_elem(p[lo:hi], g[lo:hi], m[lo:hi], v[lo:hi], k)
    return p, m, v


def sgd_step(p, g, b, items: Sequence[Item], offsets, S, m_ranks, k0, k1, lr, momentum, wd,
             nesterov, grad_scale, mask=None, found_inf=None, inplace: bool = False):
    """SGD with momentum over the buffer's tensor elements in ranks [k0, k1).
    Returns new (p, b) (the inputs themselves when inplace)."""
    if not inplace:
        p, b = p.copy(), b.copy()
    if _skip(found_inf):
        return p, b
    lr, mu, wd = F32(lr), F32(momentum), F32(wd)
    inv = F32(F32(1) / F32(grad_scale))
    for tid, r, lo, hi in fragments(items, offsets, S, m_ranks):
        if not (k0 <= r < k1) or (mask is not None and not mask[tid]):
            continue
        with np.errstate(all="ignore"):
            gg = (F32(g[lo:hi] * inv) + F32(wd * p[lo:hi])).astype(F32)
            b2 = (F32(mu * b[lo:hi]) + gg).astype(F32)
            d = (gg + F32(mu * b2)).astype(F32) if nesterov else b2
            p[lo:hi] = (p[lo:hi] - F32(lr * d)).astype(F32)
            b[lo:hi] = b2
    return p, b


def adamw8_step(p, g, m_codes, m_scales, v_codes, v_scales, specs, offsets, S, m_ranks, k0, k1,
                fmt: str, hp: dict, found_inf=None, only_tiles=None, inplace: bool = False):
    """AdamW with block-quantised moments (8-bit Adam, veScale-FSDP section
    6.3): for every tile of every quantised tensor in ranks [k0, k1):

        m = dequant(m codes, m scale);  v = dequant(v codes, v scale)
        (p, m', v') = the AdamW update above, in fp32
        m codes, m scale = block_quant(m');  v codes, v scale = block_quant(v')

    Non-quantised tensors are not touched (their fp32 moments are stepped
    with adamw_step).  Returns new (p, m_codes, m_scales, v_codes, v_scales),
    or the given arrays, written, with inplace.
    """
    from . import ops as O

    if not inplace:
        p = p.copy()
        m_codes, v_codes = m_codes.copy(), v_codes.copy()
        m_scales, v_scales = m_scales.copy(), v_scales.copy()
    if _skip(found_inf):
        return p, m_codes, m_scales, v_codes, v_scales
    k = adamw_constants(**hp)
    wanted = None if only_tiles is None else set(int(i) for i in only_tiles)
    base = 0
    for spec, l in zip(specs, offsets):
        if spec.q_rows <= 0:
            continue
        ntr, ntc = O.tile_counts(spec)
        count = ntr * ntc
        locals_ = range(count) if wanted is None else sorted(i - base for i in wanted
                                                                if base <= i < base + count)
        for idx in locals_:
            r0, r1, c0, c1 = O.tile_bounds(spec, idx)
            if not (k0 <= (l + r0 * spec.cols + c0) // S < k1):
                continue
            pos = l + (np.arange(r0, r1)[:, None] * spec.cols + np.arange(c0, c1)[None, :])
            t = base + idx
            with np.errstate(all="ignore"):
                mo = (O.decode_codes(m_codes[pos], fmt) * F32(m_scales[t])).astype(F32)
                vo = (O.decode_codes(v_codes[pos], fmt) * F32(v_scales[t])).astype(F32)
            p2, m2, v2 = adamw_elem(p[pos], g[pos], mo, vo, k)
            p[pos] = p2
            m_scales[t], m_codes[pos] = O.quant_tile(m2, fmt)
            v_scales[t], v_codes[pos] = O.quant_tile(v2, fmt)
        base += count
    return p, m_codes, m_scales, v_codes, v_scales

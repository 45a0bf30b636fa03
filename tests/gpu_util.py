"""Helpers for the GPU parity tests (device transfer, tolerance checks)."""
import numpy as np
import torch


def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda", 0)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def check_tol(got, ref, bound, rel, what=""):
    """|got - ref| <= rel * bound + 1e-6 for every element, all finite.
    Returns max(|err| / tol)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    tol = rel * np.asarray(bound, dtype=np.float64) + 1e-6
    ratio = np.abs(got - ref) / tol
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= 1.0, f"{what}: max |err|/tol = {worst:.3g} at {np.unravel_index(ratio.argmax(), ratio.shape)}"
    return worst


def guarded(n: int, dtype=torch.float32, guard: int = 64, fill=1234.5):
    """A device buffer of n elements with sentinel guard bands on both sides.
    Returns (full buffer, view of the n middle elements)."""
    full = torch.full((n + 2 * guard,), fill, dtype=dtype, device=dev())
    return full, full[guard:guard + n]


def guards_intact(full: torch.Tensor, n: int, guard: int = 64, fill=1234.5) -> bool:
    h = full.detach().cpu()
    return bool((h[:guard] == fill).all() and (h[guard + n:] == fill).all())


WS_GUARD = 4096  # bytes of sentinel before and after a guarded workspace


def guarded_ws(nbytes: int, fill: int = 0xA5):
    """A workspace of nbytes (256-byte aligned) between two sentinel bands.
    Returns (full buffer, workspace view)."""
    full = torch.full((nbytes + 2 * WS_GUARD,), fill, dtype=torch.uint8, device=dev())
    return full, full[WS_GUARD:WS_GUARD + nbytes]


def ws_guards_intact(full: torch.Tensor, nbytes: int, fill: int = 0xA5) -> bool:
    h = full.detach().cpu().numpy()
    return bool((h[:WS_GUARD] == fill).all() and (h[WS_GUARD + nbytes:] == fill).all())


def check_route_table(ws: np.ndarray, ids: np.ndarray, T: int, H: int, I: int, E: int):
    """Rebuild the routing table of moe_q4_0_decode on the host from the ids
    (a brute-force grouping by expert) and compare it with the copy the call
    left in its workspace, entry by entry (layout: include/q4moe.h,
    moe_q4_0_route_layout). Returns (vector items, matrix-core items)."""
    from moe_experts_amd import moe_q4_0_route_layout
    topk = ids.shape[1]
    io, co, mo = moe_q4_0_route_layout(T, H, I, E, topk)
    nv, nm = np.frombuffer(ws[co:co + 8].tobytes(), dtype="<i4")
    rec = np.dtype([("expert", "<i4"), ("count", "<i4"), ("res", "<i4", 2), ("pairs", "<i4", 8)])
    vit = np.frombuffer(ws[io:io + nv * rec.itemsize].tobytes(), dtype=rec)
    mit = np.frombuffer(ws[mo:mo + nm * rec.itemsize].tobytes(), dtype=rec)
    flat = ids.reshape(-1)
    per = {e: [p for p in range(flat.size) if flat[p] == e] for e in range(E)}
    exp_v = [(e, per[e]) for e in range(E) if 1 <= len(per[e]) <= 2]
    exp_m = []
    for e in range(E):
        n = len(per[e])
        if n >= 3:
            c = -(-n // 8)
            start = 0
            for i in range(c):
                sz = n // c + (1 if i < n % c else 0)
                exp_m.append((e, per[e][start:start + sz]))
                start += sz
    assert (int(nv), int(nm)) == (len(exp_v), len(exp_m)), "item counts"
    for got, (e, pairs) in list(zip(vit, exp_v)) + list(zip(mit, exp_m)):
        n = len(pairs)
        assert int(got["expert"]) == e and int(got["count"]) == n, f"expert {e} item"
        assert got["pairs"][:n].tolist() == pairs, f"expert {e} pairs"
        assert (got["pairs"][n:] == 0).all()
    valid = int(((flat >= 0) & (flat < E)).sum())
    assert sum(len(p) for _, p in exp_v + exp_m) == valid
    return exp_v, exp_m


def prefill_tile_rows() -> int:
    """Q4_MOE_PREFILL_TILE_ROWS from the C header."""
    import os
    import re
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                       "q4moe.h")
    m = re.search(r"#define\s+Q4_MOE_PREFILL_TILE_ROWS\s+(\d+)", open(hdr).read())
    return int(m.group(1))


def check_prefill_route(ws: np.ndarray, ids: np.ndarray, T: int, H: int, I: int, E: int):
    """Rebuild the stable sort of the (token, slot) pairs by expert that
    moe_q4_0_prefill leaves in its workspace (layout: include/q4moe.h,
    moe_q4_0_prefill_route_layout) with numpy's stable argsort, and compare the
    sorted rows' tokens, every pair's row, the m-tile list and the counters
    entry by entry."""
    from moe_experts_amd import moe_q4_0_prefill_route_layout
    topk = ids.shape[1]
    so, po, to, co = moe_q4_0_prefill_route_layout(T, H, I, E, topk)
    i4 = lambda off, n: np.frombuffer(ws[off:off + 4 * n].tobytes(), dtype="<i4")
    flat = ids.reshape(-1).astype(np.int64)
    vp = np.nonzero((flat >= 0) & (flat < E))[0]
    order = vp[np.argsort(flat[vp], kind="stable")]  # pair of each sorted row
    rows = np.bincount(flat[vp], minlength=E)
    R = prefill_tile_rows()
    tiles, first = [], 0
    for e in range(E):
        tiles += [(e, first + i, min(R, int(rows[e]) - i), 0) for i in range(0, int(rows[e]), R)]
        first += int(rows[e])
    ntiles, nrows = i4(co, 2)
    assert (int(ntiles), int(nrows)) == (len(tiles), order.size), "counters"
    pos = np.full(flat.size, -1, dtype=np.int64)
    pos[order] = np.arange(order.size)
    assert (i4(po, flat.size) == pos).all(), "sorted row of each pair"
    assert (i4(so, order.size) == order // topk).all(), "token of each sorted row"
    assert (i4(to, 4 * len(tiles)).reshape(-1, 4) == np.array(tiles).reshape(-1, 4)).all(), "tiles"

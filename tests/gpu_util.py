"""Helpers shared by the GPU parity tests: move BF16 bit patterns to and from the device,
run the library through its binding, compare with the FP64 oracle."""
import numpy as np
import torch

from oracle import bf16_bits_to_f64, compare


def dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 BF16 bit patterns -> contiguous bfloat16 tensor on cuda:0 (same bits)."""
    a = np.ascontiguousarray(bits).view(np.int16)
    return torch.from_numpy(a).to("cuda:0").view(torch.bfloat16)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to("cuda:0")


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of(t: torch.Tensor) -> np.ndarray:
    return bf16_bits_to_f64(bits_of(t))


def check(o_gpu, o_ref, lse_gpu=None, lse_ref=None, label=""):
    m = compare(o_gpu, o_ref, lse_gpu, lse_ref)
    print(f"[parity] {label}: rel_l2={m['rel_l2']:.3e} max_abs={m['max_abs']:.3e} "
          f"lse_max_abs={m.get('lse_max_abs', float('nan')):.3e} n={m['n_elems']}", flush=True)
    assert m["ok"], (label, m)
    return m


def device_normal_bf16(shape, seed: int) -> torch.Tensor:
    """Seeded N(0, 1) values rounded to BF16, generated on cuda:0 for inputs too large to build
    on the host. Tests copy back the rows the oracle needs, so both sides read the same bits."""
    g = torch.Generator(device="cuda:0").manual_seed(seed)
    x = torch.randn(shape, generator=g, device="cuda:0", dtype=torch.float32)
    return x.to(torch.bfloat16)


# ---- the split-KV plan of attn_fwd_splitkv, restated for choosing rows to check

def split_plan(B, H, N, slots, min_tiles=16):
    """(D, R, G, ntk) of the library's split plan (rows of 256 queries, 64-key tiles)."""
    ntq, ntk = -(-N // 256), -(-N // 64)
    items = B * H * ntq
    full, r = divmod(items, slots)
    if slots < 2 or r == 0 or ntk < min_tiles:
        return items, 0, 0, ntk
    if full >= 1:
        R, G = slots + r, slots
    else:
        R, G = items, min(slots, items * ntk // min_tiles)
        if G <= R:
            return items, 0, 0, ntk
    return items - R, R, G, ntk


def cut_tiles(B, H, N, slots):
    """Query tiles (flat index b*H*ntq + h*ntq + qt) whose key range the plan splits."""
    D, R, G, ntk = split_plan(B, H, N, slots)
    cut = set()
    for i in range(R):
        first, last = i * ntk, (i + 1) * ntk - 1
        g0 = max(g for g in range(G) if g * R * ntk // G <= first)
        g1 = max(g for g in range(G) if g * R * ntk // G <= last)
        if g0 != g1:
            cut.add(D + i)
    return cut


def cut_tile_rows(B, H, N, slots, per_tile=2, seed=0):
    """Flat rows ((b*H + h)*N + n) to check in the tiles the plan cuts: each cut tile's first and
    last valid row plus `per_tile` seeded rows inside it."""
    rng = np.random.default_rng(seed)
    ntq = -(-N // 256)
    rows = []
    for t in sorted(cut_tiles(B, H, N, slots)):
        bh, qt = divmod(t, ntq)
        lo, hi = qt * 256, min(N, (qt + 1) * 256)
        pick = {lo, hi - 1, *rng.integers(lo, hi, per_tile).tolist()}
        rows += [bh * N + n for n in pick]
    return np.array(sorted(rows), dtype=np.int64)


def device_slots() -> int:
    """Workgroups of the attention kernel that run at once on cuda:0: one per compute unit."""
    return torch.cuda.get_device_properties(0).multi_processor_count


# ---- the split-KV plan of attn_fwd_varlen_splitkv (made on the device), restated

def varlen_plan(seqlens, H, slots, min_tiles=16, sort_limit=8192):
    """(entries, D, G, cut) of the device plan: entries [(segment, query tile, key tiles)] in
    schedule order (longest segment first), D plain items, G split workgroups (0: no split) and
    the set of cut items (item = entry * H + head)."""
    lens = [int(x) for x in seqlens]
    order = sorted(range(len(lens)), key=lambda s: (-lens[s], s)) if len(lens) <= sort_limit else list(range(len(lens)))
    entries = [(s, i, -(-lens[s] // 64)) for s in order for i in range(-(-lens[s] // 256))]
    cum = [0]
    for _, _, c in entries:
        cum.append(cum[-1] + c)
    items = len(entries) * H
    cost = lambda it: entries[it // H][2]
    cum_item = lambda it: H * cum[it // H] + (it % H) * cost(it)
    r = 0
    while (r + 1) * slots <= items and cost(r * slots) == cost((r + 1) * slots - 1):
        r += 1
    D = r * slots
    if D >= items:
        return entries, items, 0, set()
    base, W = cum_item(D), H * cum[-1] - cum_item(D)
    cmax = max(c for _, _, c in entries[D // H:])
    G = min(slots, W // min_tiles)
    if G < 2 or W // G >= cmax:
        return entries, items, 0, set()

    def item_at(u):
        e = max(i for i in range(len(entries)) if H * cum[i] <= u)
        return e * H + (u - H * cum[e]) // entries[e][2]
    cut = set()
    for g in range(1, G):
        u = base + W * g // G
        it = item_at(u)
        if u != cum_item(it):
            cut.add(it)
    return entries, D, G, cut


def varlen_cut_rows(seqlens, H, slots, per_item=2, seed=0):
    """Flat rows h * T + t in the items the plan cuts: each cut item's first and last row plus
    `per_item` seeded rows (LSE layout [H, T])."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in seqlens]
    starts = np.concatenate([[0], np.cumsum(lens)])
    T = int(starts[-1])
    entries, _, _, cut = varlen_plan(lens, H, slots)
    rows = set()
    for it in cut:
        s, i, _ = entries[it // H]
        h = it % H
        lo, hi = i * 256, min(lens[s], (i + 1) * 256)
        for r in {lo, hi - 1, *rng.integers(lo, hi, per_item).tolist()}:
            rows.add(h * T + int(starts[s]) + r)
    return np.array(sorted(rows), dtype=np.int64)


def dominated_dense(N, H=2, seed=31, vmax=7.0):
    """Host BF16 bits [1, H, N, 128] of rows that one key dominates: K = Q, so each query's own
    key has logit |q|^2/sqrt(128) (about 11, weight about 0.98 over the N(0,1) logits of the
    others), and V ~ 2.5 N(0,1) clipped to +-vmax, so many outputs sit in [4, 8) where half a
    BF16 ulp is 0.0156. Dividing by the FP32 sum alone leaves the dominant key's BF16 rounding
    (up to 2^-8 of |v|) on top of that and misses the 2e-2 bar (a CPU replay of the key loop
    on this case: 0.038); the kernel's corrected normaliser does not."""
    from oracle import bf16_bits_to_f64
    from workloads import f32_to_bf16_bits, random_dense
    qb, _, _ = random_dense(1, H, N, seed=seed)
    _, _, vb = random_dense(1, H, N, seed=seed + 1)
    v = np.clip(bf16_bits_to_f64(vb) * 2.5, -vmax, vmax)
    return qb, qb.copy(), f32_to_bf16_bits(v.astype(np.float32))

"""A CPU model of the engine's per-workgroup hand-offs on the attention path.

Three stages of a layer do not wait for every workgroup of the stage before
them; they wait on the completion flags of exactly the workgroups they read
from:
  * an attention unit (head group g, position chunk c, run by workgroup
    g * nch + c) waits for the q_b workgroups from the owner of the group's
    first query row to the owner of its last (split_owner), and reads the
    group's q_lat partial slots and rotary queries;
  * a W_UV workgroup waits for the attention units of the head groups its
    rows fall in, and reads those heads' chunk partials.
The model recomputes, by brute force over every workgroup's row share
(floor(ng * w / G) * gran .. of ng = rows / gran row groups, the planner's
split), which workgroups write each piece of data, and checks that every
writer of what a consumer reads lies inside the flag range the consumer waits
on, that the flag ranges use the closed-form owner the kernel uses, and that
the q_lat slots a unit adds are exactly the ones q_b workgroups write. Shapes:
the DeepSeek-V3 layer, the small and the ragged models, on several
workgroup counts (more and fewer workgroups than heads, counts that do not
divide the rows). Pure Python: no GPU, no library."""
import pytest

from synth import configs


def split_rows(rows, gran, G, w):
    ng = rows // gran
    return ng * w // G * gran, ng * (w + 1) // G * gran


def split_owner(rows, gran, G, r):
    """The kernel's closed form for the workgroup whose share holds row r."""
    ng, g = rows // gran, r // gran
    return ((g + 1) * G + ng - 1) // ng - 1


def unit_rows(kbytes):
    return 1024 // kbytes if kbytes < 1024 and kbytes & (kbytes - 1) == 0 else 1


def attn_chunks(nch_plan, ctx, chunk_pos=64):
    return min(nch_plan, max(1, (ctx + chunk_pos - 1) // chunk_pos))


def plan_shape(cfg, G, max_ctx):
    H, qkh = cfg.n_heads, cfg.qk_nope + cfg.rope
    hg = 16 if H % 16 == 0 else 8
    n_hg = H // hg
    nch = min(G // n_hg, max(1, (max_ctx + 15) // 16), 64)
    return {"H": H, "qkh": qkh, "hg": hg, "n_hg": n_hg, "nch": nch, "qb_gran": max(2, unit_rows(cfg.q_lora)),
            "uv_gran": unit_rows(cfg.kv_lora)}


def qb_writers(cfg, p, G):
    """Brute force: per head, the q_b workgroups that write a q_lat partial
    (own a nope row) and those that write its rotary queries (own a rotary
    row). Also checks that a rotary pair never straddles two workgroups."""
    H, qkh, dn, gran = p["H"], p["qkh"], cfg.qk_nope, p["qb_gran"]
    lat = {h: set() for h in range(H)}
    rot = {h: set() for h in range(H)}
    for w in range(G):
        ra, rb = split_rows(H * qkh, gran, G, w)
        for r in range(ra, rb):
            h, j = divmod(r, qkh)
            if j < dn:
                lat[h].add(w)
            else:
                rot[h].add(w)
                if (j - dn) % 2 == 0:
                    assert r + 1 < rb, f"rotary pair at row {r} split between workgroups"
    return lat, rot


def check_attention(cfg, G, max_ctx, owner=split_owner):
    p = plan_shape(cfg, G, max_ctx)
    H, qkh, hg, gran = p["H"], p["qkh"], p["hg"], p["qb_gran"]
    lat, rot = qb_writers(cfg, p, G)
    rows = H * qkh
    for grp in range(p["n_hg"]):
        wlo = owner(rows, gran, G, grp * hg * qkh)
        whi = owner(rows, gran, G, (grp + 1) * hg * qkh - 1)
        for h in range(grp * hg, (grp + 1) * hg):
            writers = lat[h] | rot[h]
            assert writers and all(wlo <= w <= whi for w in writers), \
                f"group {grp} head {h}: writers {sorted(writers)} outside flags [{wlo}, {whi}]"
            # the unit adds slots k of the head's partials, workgroup first + k, over the
            # planner's span first .. owner of the last nope row; the slots actually
            # written are exactly the nope-row owners
            first = owner(rows, gran, G, h * qkh)
            last = owner(rows, gran, G, h * qkh + cfg.qk_nope - 1)
            assert lat[h] <= set(range(first, last + 1))
            assert min(lat[h]) == first and max(lat[h]) == last
            for w in range(first, last + 1):
                ra, rb = split_rows(rows, gran, G, w)
                assert (rb > ra) == (w in lat[h]), f"head {h}: slot of workgroup {w} read but not written"
    return p


def check_uv(cfg, G, max_ctx, ctx):
    p = plan_shape(cfg, G, max_ctx)
    H, hg, dv = p["H"], p["hg"], cfg.v_head
    nch = attn_chunks(p["nch"], ctx)
    units = p["n_hg"] * nch
    assert units <= G
    # attention partial writers: unit u = grp * nch + ch writes heads of grp, chunk ch
    part_writers = {h: {(h // hg) * nch + ch for ch in range(nch)} for h in range(H)}
    for w in range(G):
        ra, rb = split_rows(H * dv, p["uv_gran"], G, w)
        if ra >= rb:
            continue
        h0, h1 = ra // dv, (rb - 1) // dv
        lo, hi = h0 // hg * nch, (h1 // hg + 1) * nch - 1
        for h in range(h0, h1 + 1):
            assert all(lo <= u <= hi for u in part_writers[h]), (w, h)
            assert all(u < units for u in part_writers[h])


CASES = [("dsv3_moe_layer", G) for G in (256, 240, 304, 128, 200)] + \
        [("tiny", G) for G in (256, 40, 16, 9)] + [("ragged", G) for G in (256, 67, 96, 33)]


@pytest.mark.parametrize("name,G", CASES)
def test_attention_waits_cover_their_writers(name, G):
    cfg = configs.get(name)
    p = plan_shape(cfg, G, 9216)
    if p["n_hg"] > G:
        pytest.skip("fewer workgroups than head groups (the planner rejects it)")
    check_attention(cfg, G, 9216)
    for ctx in (1, 64, 65, 1025, 2048, 9216):
        check_uv(cfg, G, 9216, ctx)


def test_model_catches_an_owner_off_by_one():
    """A flag range from an owner one workgroup too early misses the last
    q_b workgroup of some head group."""
    cfg = configs.get("dsv3_moe_layer")
    early = lambda rows, gran, G, r: split_owner(rows, gran, G, r) - (1 if r % 7 == 6 else 0)  # noqa: E731
    with pytest.raises(AssertionError):
        check_attention(cfg, 240, 9216, owner=early)


def test_split_owner_inverts_split_rows():
    for rows, gran, G in ((24576, 2, 256), (24576, 2, 240), (512, 2, 9), (4608, 2, 67), (16384, 1, 304)):
        for w in range(G):
            ra, rb = split_rows(rows, gran, G, w)
            for r in range(ra, rb):
                assert split_owner(rows, gran, G, r) == w

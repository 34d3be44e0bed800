"""Python statement of the documented work-split rule (pa_set_work_split in
include/pa_decode.h), used to predict the library's plan in the tests."""

MAX_SHIFT = 4
MAX_SLOTS = 1024
MAX_GRID = 1 << 24


def max_piece_shift(P):
    """log2 of the most pieces (<= 16, each a multiple of 64 tokens) P divides into."""
    if P <= 0 or P % 64:
        return 0
    m, sh = P // 64, 0
    while sh < MAX_SHIFT and m % 2 == 0:
        m //= 2
        sh += 1
    return sh


def piece_slots(items, P):
    sh = max_piece_shift(P)
    return min(MAX_SLOTS, items << sh) if sh else 0


def plan(items, P, pieces, first_item=0, ncu=None):
    """(first cut item, pieces per cut item, work-groups) for a V2 launch."""
    msh = max_piece_shift(P)
    none = (items, 1, items)
    if msh == 0 or pieces in (0, 1) or items == 0:
        return none
    if pieces > 1:
        shift = min(pieces.bit_length() - 1, msh)
        first = min(max(first_item, 0), items)
    else:
        if items < ncu:
            shift = min((2 * ncu // items).bit_length() - 1, msh)
            first = 0
        else:
            rem = items % ncu
            if rem == 0 or 2 * rem > ncu:
                return none
            first = items - rem
            shift = 0
            for s in range(1, msh + 1):
                if rem << s > piece_slots(items, P):
                    break
                shift = s
                if (rem << s) % ncu == 0:
                    break
    if shift <= 0:
        return none
    first = max(first, items - (piece_slots(items, P) >> shift))
    if first >= items:
        return none
    wgs = first + ((items - first) << shift)
    if wgs > MAX_GRID:
        return none
    return first, 1 << shift, wgs

"""Reader for the small text fixtures in this folder (masks and tile maps)."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def read_blocks(name):
    """Return {block_name: (header_tokens, [[int,...], ...])} from a fixture file."""
    blocks = {}
    cur = None
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tok = line.split()
            if tok[0] in ("mask", "skipped_tiles"):
                key = (tok[0], tok[1])
                blocks[key] = (tok[2:], [])
                cur = blocks[key][1]
            else:
                cur.append([int(t) for t in tok])
    return blocks

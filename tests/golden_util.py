import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def philox_kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            v = [int(x, 16) for x in line.split()]
            rows.append((v[0:4], v[4:6], v[6:10]))
    return rows

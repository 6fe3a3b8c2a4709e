"""Write moe64_counts_seed0.txt from the routing generator (datagen only)."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import datagen  # noqa: E402

r = datagen.moe_route(datagen.MOE["moe64"])
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "moe64_counts_seed0.txt")
head = open(path).read().split("\n")[:5] if os.path.exists(path) else []
with open(path, "w") as f:
    f.write("\n".join(l for l in head if l.startswith("#")) + "\n")
    f.write(" ".join(str(int(c)) for c in r.counts) + "\n")

"""Runs the nine-step walkthrough fixture against any tree with the Python
tree API (the oracle or the native library)."""
import os

from tests import radix_ops

HERE = os.path.dirname(os.path.abspath(__file__))
SIZES = dict(S=8, A1=8, A2=8, A3=8, B1=8, B2=8, E=16, Q1=4, Q2=4, Q3=4,
             X1=4, X2=4, X3=4, X4=4)


def blocks():
    out, base = {}, 100
    for name, n in SIZES.items():
        out[name] = list(range(base, base + n))
        base += 100
    return out


def load_steps():
    steps = []
    with open(os.path.join(HERE, "golden", "radix_walkthrough.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            cols = [c.strip() for c in line.split("|")]
            def lst(c):
                return [] if c == "-" else c.split(",")
            steps.append(dict(step=int(cols[0]), reqs=lst(cols[1]), ballast=int(cols[2]),
                              matched=[int(x) for x in lst(cols[3])], added=lst(cols[4]),
                              evicted=lst(cols[5]), free=int(cols[6])))
    return steps


def run(make_tree):
    B = blocks()

    def label_name(label):
        # split a label into whole blocks
        parts, i = [], 0
        while i < len(label):
            for nm, toks in B.items():
                if label[i:i + len(toks)] == toks:
                    parts.append(nm); i += len(toks); break
            else:
                raise AssertionError(f"label {label} is not made of whole blocks")
        return ".".join(parts)

    def seq(spec):
        return [t for nm in spec.split(".") for t in B[nm]]

    tree = make_tree(64)
    for st in load_steps():
        before = radix_ops.parse_dump(tree.serialize())
        ids_before = {nd["id"]: nd for nd in before}
        held = []
        if st["ballast"]:
            code, held = tree.alloc(st["ballast"])
            assert code == 0
        stream = []
        if st["reqs"]:
            seqs = [seq(r) for r in st["reqs"]]
            code, tb = tree.batch_prepare(seqs)
            assert code == 0, (st["step"], code)
            assert list(tb["prefix_lens"]) == st["matched"], st
            stream = list(tb["new_slots"])
            assert tree.batch_commit(seqs, tb["req_to_token"], tb["nodes"]) == 0
        # the free list is FIFO: the slots this step popped, then what is left,
        # give the order in which evicted nodes' slots were appended
        stream += tree.free_list()
        after = radix_ops.parse_dump(tree.serialize())
        ids_after = {nd["id"] for nd in after}
        added = sorted(label_name(nd["label"]) for nd in after if nd["id"] not in ids_before)
        assert added == sorted(st["added"]), (st["step"], added)
        gone = [i for i in ids_before if i not in ids_after]
        order = sorted((stream.index(ids_before[nid]["slots"][0]), label_name(ids_before[nid]["label"]))
                       for nid in gone)
        evicted = [nm for _, nm in order]
        assert evicted == st["evicted"], (st["step"], evicted)
        if held:
            assert tree.free(held) == 0
        assert len(tree.free_list()) == st["free"], (st["step"], len(tree.free_list()))
    return tree

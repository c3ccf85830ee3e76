"""Write closed_forms.txt: selected-token log-probabilities with a closed form.

The operator is the log-softmax of the logits evaluated at the target
("Announcing RL-Kernel for vime", section "Key Capabilities").  Two input
families have exact answers:

* all logits equal (h = 0 or W = 0):      logp = -ln V for every target;
* one-hot logits z_v = alpha * [v == v0]: logp(v0)    = -log1p((V-1) e^-alpha)
                                          logp(v!=v0) = -alpha - log1p((V-1) e^-alpha)

This script uses Python's math module only (no oracle, no GPU).
Run:  python tests/golden/make_closed_forms.py
"""
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def rows():
    for V in (4096, 151936):
        yield ("uniform", V, 0.0, "any", -math.log(V))
        for alpha in (1.0, 8.0, 40.0):
            c = math.log1p((V - 1) * math.exp(-alpha))
            yield ("onehot", V, alpha, "target", -c)
            yield ("onehot", V, alpha, "other", -alpha - c)


def main():
    with open(os.path.join(HERE, "closed_forms.txt"), "w") as f:
        f.write("# kind V alpha which expected_logp   (see make_closed_forms.py for the formulas)\n")
        for kind, V, alpha, which, val in rows():
            f.write(f"{kind} {V} {alpha!r} {which} {val!r}\n")


if __name__ == "__main__":
    main()

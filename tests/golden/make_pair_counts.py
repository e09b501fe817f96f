"""Writes pair_counts.txt: selected (query, key) pair counts of static masks,
evaluated from closed forms by integer arithmetic alone (no oracle, no GPU).

  * A-shape (MInference 1.0 summary page, "Approach": a sink of the first
    tokens plus a local window): row i keeps min(i + 1, w) window keys and
    max(0, min(s, i + 1 - w)) sink keys outside the window.  The sum over
    rows splits into the rows inside the first window, w (w + 1) / 2, and
    the rest, (L - w) w plus the sink terms 1 + 2 + ... + s and (L - w - s) s.
  * Parallel encoding (PEVLM verdict page, key_machinery): the page's
    operation count over whole blocks, per unit of its factor 2H, is
    S^2 + Q^2 + N B^2 + Q S + N Q B + N S B for a sink of S tokens, N context
    blocks of B tokens and a question of Q tokens.  A causal prefill drops the
    strict upper triangle of each diagonal block (sink, contexts, question).

Run from the repository root:  python tests/golden/make_pair_counts.py
"""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def ashape(L, s, w):
    assert L >= w + s
    return w * (w + 1) // 2 + (L - w) * w + s * (s + 1) // 2 + (L - w - s) * s


def parallel(S, B, N, Q):
    page = S * S + Q * Q + N * B * B + Q * S + N * Q * B + N * S * B
    upper = S * (S - 1) // 2 + N * (B * (B - 1) // 2) + Q * (Q - 1) // 2
    return page - upper


ROWS = [("ashape", 4096, 64, 512), ("ashape", 3000, 17, 900), ("ashape", 1000, 0, 1),
        ("ashape", 131072, 128, 4096)]
PAR = [(64, 48, 5, 30), (0, 37, 4, 0), (100, 64, 3, 64), (7, 1, 9, 5), (50, 20, 0, 40), (0, 90, 1, 0),
       (196, 392, 6, 128)]


def main():
    lines = ["# kind L sink window_or_block n_blocks question pairs",
             "# written by make_pair_counts.py from closed forms (see its docstring)"]
    for kind, L, s, w in ROWS:
        lines.append(f"ashape {L} {s} {w} 0 0 {ashape(L, s, w)}")
    for S, B, N, Q in PAR:
        lines.append(f"parallel {S + N * B + Q} {S} {B} {N} {Q} {parallel(S, B, N, Q)}")
    with open(os.path.join(HERE, "pair_counts.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()

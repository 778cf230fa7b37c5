"""Markdown summary of a parity log (the JSON lines the bf16 whole-step
comparisons append to the file SLT_PARITY_LOG names).

    python tests/parity_summary.py <log.jsonl>

Per case: the largest normwise error, 99.9th percentile, worst band ratio and
fraction of elements beyond their band over the case's gradient tensors (the
tensor named), the same for the oracle's companion where the case computed
it, and the exempt (sign-tie) weights against the reference's own tie set."""
import collections
import json
import sys


def short(t):
    for pre in ("grad ", "accumulated "):
        if t.startswith(pre):
            return t[len(pre):]
    return t


def main(path):
    rows = [json.loads(l) for l in open(path)]
    by = collections.OrderedDict()
    for r in rows:
        by.setdefault(r["case"], []).append(r)
    print("| case | tensors | max normwise | max 99.9 % | worst (bands) | max fraction beyond | "
          "companion normwise / worst / fraction | exempt weights (reference ties) |")
    print("|---|---:|---|---|---|---|---|---|")
    for case, rs in by.items():
        g = [r for r in rs if "normwise" in r]
        w = [r for r in rs if "exempt" in r]
        if not g:
            continue
        top = lambda k: max(g, key=lambda r: r[k])
        nw, q, wo, fr = top("normwise"), top("q999"), top("worst"), top("frac")
        comp = "—"
        if any("comp_normwise" in r for r in g):
            c = [r for r in g if "comp_normwise" in r]
            comp = (f"{max(r['comp_normwise'] for r in c):.2e} / {max(r['comp_worst'] for r in c):.2f} / "
                    f"{max(r['comp_frac'] for r in c):.1e}")
        ex = "—"
        if w:
            n = sum(r["n"] for r in w)
            ex = f"{sum(r['exempt'] for r in w) / n:.1%} ({sum(r['exempt_ref'] for r in w) / n:.1%})"
        print(f"| {case} | {len(g)} | {nw['normwise']:.2e} ({short(nw['tensor'])}) | {q['q999']:.2f} | "
              f"{wo['worst']:.2f} ({short(wo['tensor'])}) | {fr['frac']:.1e} ({short(fr['tensor'])}) | {comp} | {ex} |")


if __name__ == "__main__":
    main(sys.argv[1])

"""Product text restates the pages and never quotes them: no source file, header,
oracle file or design note shares a run of words with the pages' text beyond the
titles and section names that cite them.  Runs where the pages' text is present
(it is not on every machine); skipped elsewhere."""
from __future__ import annotations

import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
PAGES = Path("/root/reference/PAPER.md")

# Citations: page titles, section names and a file path, which the sources name
# on purpose.
CITED = [
    "Issue #323 [WS2][Logprob] H100 validation and reproduction guide for Issue #241 PR1-PR5",
    "PR #289 [WS2][PR4][Logp] feat: add distributed TP/CP logprob drift report",
    "H100 canonical TP/CP validation",
    "2. Six-Case TP/CP Matrix",
    "4. Cross-Topology Bitwise Check",
    "docs/usage/h100-matrix-validation.md",
]


def words(text: str) -> list[str]:
    return re.findall(r"[a-z0-9_]+", text.lower())


def overlaps(text: str, shingles: set, n: int, allowed: list[str]) -> list[str]:
    w = words(text)
    hits = [i for i in range(len(w) - n + 1) if tuple(w[i:i + n]) in shingles]
    runs, out = [], []
    for h in hits:
        if runs and h <= runs[-1][1] + 1:
            runs[-1][1] = h
        else:
            runs.append([h, h])
    for a, b in runs:
        run = " ".join(w[a:b + n])
        if all(re.fullmatch(r"\d+e?", t) for t in w[a:b + n]):
            continue  # printed values (the golden fixtures cite them)
        if not any(run in c for c in allowed):
            out.append(run)
    return out


@pytest.mark.skipif(not PAGES.exists(), reason="the pages' text is not on this machine")
def test_no_quoted_runs_of_the_pages():
    pw = words(PAGES.read_text(errors="ignore"))
    allowed = [" ".join(words(c)) for c in CITED]
    found = []
    # prose-heavy files: runs of 6 words; Python: 8 (short code idioms such as
    # subprocess keyword lists also occur in the pages' listings)
    groups = [
        (6, list((ROOT / "vocab_selected_token_amd" / "csrc").glob("*")) +
         list((ROOT / "include").glob("*.h")) + list((ROOT / "oracle").glob("*.c")) +
         [ROOT / "DESIGN.md", ROOT / "README.md"] + list((ROOT / "tests" / "golden").glob("*"))),
        (8, list(ROOT.glob("*.py")) + list((ROOT / "vocab_selected_token_amd").glob("*.py")) +
         list((ROOT / "oracle").glob("*.py")) + list((ROOT / "tests").glob("*.py"))),
    ]
    for n, files in groups:
        shingles = {tuple(pw[i:i + n]) for i in range(len(pw) - n + 1)}
        for f in files:
            if f.is_file() and f.suffix in (".c", ".h", ".hip", ".cpp", ".py", ".md", ".txt"):
                for run in overlaps(f.read_text(errors="ignore"), shingles, n, allowed):
                    found.append(f"{f.relative_to(ROOT)}: {run}")
    assert not found, "text repeated from the pages:\n" + "\n".join(found)

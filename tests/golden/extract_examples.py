"""Transcribe the worked examples printed on the operator pages into JSON fixtures.

This recipe reads a plain-text extraction of the operator pages (the path is
its one argument) and writes one JSON file per operator next to this script:

  matmul_examples.json         ONNX MatMul (onnx-light docs), "Examples" section
  gemm_examples.json           ONNX Gemm (onnx-light docs), "Examples" section
  qlinearmatmul_examples.json  QLinearMatMul - version 10 (onnx-light rst), "Examples"
  groupedmatmul_examples.json  GroupedMatMul - 29 (onnx.ai), "Examples" (inputs only:
                               the page computes the outputs with a helper whose body
                               it does not print)

Numbers are copied as the printed tokens (strings), so a test can derive the
printed precision of each value. Nothing here is evaluated: the GroupedMatMul
snippets are parsed with `ast.literal_eval` on list literals plus a few regexes
for `np.arange(...).reshape(...)`, `np.zeros(...)` and `np.empty(...)`.

Run:  python tests/golden/extract_examples.py PAGE_TEXT_FILE
"""
import ast
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))

NUM = re.compile(r"[-+]?(?:\d+\.?\d*|\.\d+)(?:[eE][-+]?\d+)?")
FIELD = re.compile(r"(\w+): shape=\(([^)]*)\), dtype=(\w+)")


def _shape(txt):
    return [int(s) for s in txt.replace(" ", "").split(",") if s != ""]


def _count(shape):
    n = 1
    for s in shape:
        n *= s
    return n


def _split_pages(text):
    parts = re.split(r"=-=-= page (\d) of 5: (\S+) =-=-=", text)
    pages = {}
    for i in range(1, len(parts), 3):
        pages[int(parts[i])] = (parts[i + 1], parts[i + 2])
    return pages


def _parse_fields(block):
    """Parse 'name: shape=(..), dtype=..' fields followed by printed values."""
    out = {}
    ms = list(FIELD.finditer(block))
    for j, m in enumerate(ms):
        end = ms[j + 1].start() if j + 1 < len(ms) else len(block)
        body = block[m.end():end]
        # stop at section words that follow the last field of a group
        body = re.split(r"Outputs:|\.\. code-block::|\*\*test_cc|Differences with", body)[0]
        shape = _shape(m.group(2))
        toks = NUM.findall(body)
        n = _count(shape)
        if len(toks) < n:
            raise ValueError("field %s: expected %d values, found %d" % (m.group(1), n, len(toks)))
        out[m.group(1)] = {"shape": shape, "dtype": m.group(3), "text": toks[:n]}
    return out


def _split_io(block):
    i = block.index("Inputs:")
    o = block.index("Outputs:")
    return block[:i], block[i:o], block[o:]


def parse_matmul_or_gemm(page_text, prefix, title):
    heads = list(re.finditer(r"^(" + prefix + r"\w+)\s*$", page_text, re.M))
    examples = []
    for j, h in enumerate(heads):
        end = heads[j + 1].start() if j + 1 < len(heads) else page_text.find("Differences with")
        block = page_text[h.end():end]
        head, ins, outs = _split_io(block)
        attrs = {}
        for am in re.finditer(r"^(transA|transB|alpha|beta) = (\S+)\s*$", head, re.M):
            attrs[am.group(1)] = am.group(2)
        examples.append({
            "name": h.group(1),
            "cite": "%s, Examples: %s" % (title, h.group(1)),
            "attrs": attrs,
            "inputs": _parse_fields(ins),
            "outputs": _parse_fields(outs),
        })
    return examples


def parse_qlinear(page_text, title):
    parts = re.split(r"\*\*(test_cc_qlinearmatmul_\w+)\*\*", page_text)
    examples = []
    for i in range(1, len(parts), 2):
        name, block = parts[i], parts[i + 1]
        _, ins, outs = _split_io(block)
        examples.append({
            "name": name,
            "cite": "%s, Examples: %s" % (title, name),
            "attrs": {},
            "inputs": _parse_fields(ins),
            "outputs": _parse_fields(outs),
        })
    return examples


def _np_value(expr, dtype_names):
    """Parse the few numpy constructor forms the GroupedMatMul page uses."""
    expr = expr.strip()
    m = re.match(r"np\.array\(\s*(.*?),\s*dtype=([\w.]+)\s*,?\s*\)$", expr, re.S)
    if m:
        data = ast.literal_eval(m.group(1))
        flat, shape = [], []

        def walk(x, depth):
            if isinstance(x, list):
                if len(shape) <= depth:
                    shape.append(len(x))
                for e in x:
                    walk(e, depth + 1)
            else:
                flat.append(x)
        walk(data, 0)
        return {"shape": shape, "dtype": dtype_names(m.group(2)), "values": flat}
    m = re.match(r"np\.arange\((\d+), dtype=([\w.]+)\)\.reshape\(([\d, ]+)\)$", expr)
    if m:
        n = int(m.group(1))
        return {"shape": _shape(m.group(3)), "dtype": dtype_names(m.group(2)),
                "values": "arange", "count": n}
    m = re.match(r"np\.(zeros|empty)\(\(([\d, ]+)\), dtype=([\w.]+)\)$", expr)
    if m:
        shape = _shape(m.group(2))
        return {"shape": shape, "dtype": dtype_names(m.group(3)),
                "values": [0] * _count(shape) if m.group(1) == "zeros" else []}
    raise ValueError("unparsed numpy expression: " + expr)


def parse_grouped(page_text, title):
    secs = re.split(r"^#### (_?\w+)\s*$", page_text, flags=re.M)
    examples = []
    for i in range(1, len(secs), 2):
        sec, body = secs[i], secs[i + 1]
        code = body.split("```python", 1)[1].split("```", 1)[0]
        node_inputs = re.search(r"inputs=\[([^\]]*)\]", code).group(1)
        inputs = [s.strip().strip('"') for s in node_inputs.split(",")]
        loop_dtypes = re.search(r"for dtype in \(([^)]*)\)", code)
        loop_idx = re.search(r"for index_dtype in \(([^)]*)\)", code)

        def dtype_names(tok):
            tok = tok.replace("np.", "")
            return {"dtype": "T", "index_dtype": "Tind"}.get(tok, tok)

        vals = {}
        for name in ("input", "weights", "group_indices", "bias"):
            m = re.search(r"^\s*" + name + r" = (np\..*?)\n(?=\s*\w+ = |\s*output = )", code, re.M | re.S)
            if m:
                vals[name] = _np_value(" ".join(m.group(1).split()), dtype_names)
        ex = {
            "name": sec,
            "cite": "%s, Examples: %s" % (title, sec),
            "node_inputs": inputs,
            "inputs": vals,
        }
        if loop_dtypes:
            ex["T_values"] = [t.strip().replace("np.", "") for t in loop_dtypes.group(1).split(",") if t.strip()]
        if loop_idx:
            ex["Tind_values"] = [t.strip().replace("np.", "") for t in loop_idx.group(1).split(",") if t.strip()]
        examples.append(ex)
    return examples


def main(argv):
    if len(argv) != 2:
        print("usage: extract_examples.py PAGE_TEXT_FILE", file=sys.stderr)
        return 2
    with open(argv[1], encoding="utf-8") as f:
        text = f.read()
    pages = _split_pages(text)
    t1 = "ONNX MatMul (onnx-light operator docs, since version 13)"
    t3 = "ONNX Gemm (onnx-light operator docs, since version 13)"
    t4 = "QLinearMatMul - version 10 (onnx-light operator docs)"
    t5 = "GroupedMatMul - 29 (onnx.ai operator docs)"
    sets = {
        "matmul_examples.json": parse_matmul_or_gemm(pages[1][1], "test_cc_matmul_", t1),
        "gemm_examples.json": parse_matmul_or_gemm(pages[3][1], "test_cc_gemm_", t3),
        "qlinearmatmul_examples.json": parse_qlinear(pages[4][1], t4),
        "groupedmatmul_examples.json": parse_grouped(pages[5][1], t5),
    }
    srcs = {"matmul_examples.json": pages[1][0], "gemm_examples.json": pages[3][0],
            "qlinearmatmul_examples.json": pages[4][0], "groupedmatmul_examples.json": pages[5][0]}
    for fn, exs in sets.items():
        doc = {"source_page": srcs[fn], "count": len(exs), "examples": exs}
        with open(os.path.join(HERE, fn), "w") as f:
            json.dump(doc, f, indent=1)
        print("%s: %d examples" % (fn, len(exs)))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))

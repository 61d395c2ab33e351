"""Plant plausible mistakes in copies of the CPU oracle (on the CPU only; a
mistake goes into every place its expression appears) and check that the
pins catch every one: a dropped term, a wrong sign, a wrong or
transposed index, a missing bias, cap or mask.  Each mutant must fail at least
one pin in tests/oracle_pins.py.  (Equivalent mutants, such as taking the
softmax shift from the minimum instead of the maximum, change no result and
are not listed.)"""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = [
    ("offsets drop the running sum",
     "offsets[i + 1] = offsets[i] + (int64_t)lengths[i];", "offsets[i + 1] = (int64_t)lengths[i];"),
    ("floor mod takes |r|", "if (r < 0) r += n;", "if (r < 0) r = -r;"),
    ("truncating mod", "if (r < 0) r += n;", "(void)n;"),
    ("hash search off by one", "if (sorted_keys[mid] < key) lo = mid + 1;",
     "if (sorted_keys[mid] <= key) lo = mid + 1;"),
    ("hash miss reads slot 0", "if (r < 0) continue;                 /* hash miss",
     "if (r < 0) r = 0;                 /* hash miss"),
    ("pool from the wrong table", "int64_t r = orc_resolve(&tables[k], values[offsets[bag] + i]);",
     "int64_t r = orc_resolve(&tables[0], values[offsets[bag] + i]);"),
    ("pool drops the last id",
     "for (int64_t i = 0; i < lengths[bag]; ++i) {\n                int64_t r = orc_resolve(",
     "for (int64_t i = 0; i + 1 < lengths[bag]; ++i) {\n                int64_t r = orc_resolve("),
    ("q - s sign flipped", "x[96 + c] = qc - sc;", "x[96 + c] = sc - qc;"),
    ("q * s replaced by q + s", "x[144 + c] = qc * sc;", "x[144 + c] = qc + sc;"),
    ("q and s blocks swapped", "x[c] = qc;\n                x[48 + c] = sc;",
     "x[c] = sc;\n                x[48 + c] = qc;"),
    ("W1 read transposed", "a += w1[o * 192 + i] * x[i];", "a += w1[i * 256 + o] * x[i];"),
    ("b1 dropped", "double a = b1[o];", "double a = 0.0;"),
    ("b2 dropped", "double a = b2[o];", "double a = 0.0;"),
    ("b3 dropped", "double a = b3;", "double a = 0.0;"),
    ("no ReLU after 64", "h2[o] = a > 0.0 ? a : 0.0;", "h2[o] = a;"),
    ("no ReLU after 256", "h1[o] = a > 0.0 ? a : 0.0;", "h1[o] = a;"),
    ("softmax denominator without max shift", "den += exp(e[j] - m);", "den += exp(e[j]);"),
    ("cap one short of max_len", "int64_t L = seq_lengths[b] < max_len ? seq_lengths[b] : max_len;",
     "int64_t L = seq_lengths[b] < max_len ? seq_lengths[b] : max_len - 1;"),
    ("sub-feature rows reversed", "orc_emb(&seq_tables[f], raw, sj + j * 48 + f * 16);",
     "orc_emb(&seq_tables[f], raw, sj + j * 48 + (2 - f) * 16);"),
    ("sequence position off by one", "int64_t raw = seq_values[f * seq_stride + seq_offsets[b] + j];",
     "int64_t raw = seq_values[f * seq_stride + seq_offsets[b] + (j > 0 ? j - 1 : 0)];"),
    ("weighted sum uses x not s", "out[c] += p * sj[j * 48 + c];", "out[c] += p * x[c];"),
    ("weights not normalised", "double p = exp(e[j] - m) / den;", "double p = exp(e[j] - m);"),
    ("tower layers without ReLU", "out[o] = acc > 0.0 ? acc : 0.0;", "out[o] = acc;"),
    ("tower weights read transposed", "acc += W[(int64_t)o * nin + i] * in[i];",
     "acc += W[(int64_t)i * nout + o] * in[i];"),
    ("tower biases dropped", "double acc = bias[o];", "double acc = 0.0;"),
    ("deep rows read at stride 256", "pooled + s * ld, 256, 512, d1);",
     "pooled + s * 256, 256, 512, d1);"),
    ("attention output left out of the concat", "z[128 + c] = att[s * 48 + c];",
     "z[128 + c] = 0.0;"),
    ("attention written over the deep output", "z[128 + c] = att[s * 48 + c];",
     "z[c] = att[s * 48 + c];"),
    ("logit bias dropped", "double lg = bo, mag", "double lg = 0.0, mag"),
    ("logit scale drops the bias", "mag = fabs(bo);", "mag = 0.0;"),
    ("logistic sign flipped", "prob[s] = 1.0 / (1.0 + exp(-lg));", "prob[s] = 1.0 / (1.0 + exp(lg));"),
    ("deep tower skips its last layer", "orc_layer(wd3, bd3, d2, 256, 128, z);",
     "for (int c = 0; c < 128; ++c) z[c] = d2[c];"),
    ("insert probes every other slot", "at = (at + 1 == capacity) ? 0 : at + 1;",
     "at = (at + 2 >= capacity) ? 0 : at + 2;"),
    ("insert probe does not wrap", "at = (at + 1 == capacity) ? 0 : at + 1;",
     "at = (at + 1 == capacity) ? at : at + 1;"),
    ("home slot by modulo", "return (int64_t)(((u128)h * (u128)(uint64_t)capacity) >> 64);",
     "return (int64_t)(h % (uint64_t)capacity);"),
    ("digest keeps a zero byte", "return d ? d : 1;", "return d;"),
    ("assign stores a second copy", "if (tkeys[at] == key) { slot = at; break; }",
     "if (0) { slot = at; break; }"),
    ("LFU overwrites the count", "tscores[slot] = tscores[slot] + 1;", "tscores[slot] = 1;"),
    ("STEP score not written", "if (mode == ORC_SCORE_STEP) tscores[slot] = step;",
     "if (0) tscores[slot] = step;"),
    ("check ignores holes on the path", "if (tkeys[q] == ORC_EMPTY_KEY) { ++bad; break; }",
     "if (0) { ++bad; break; }"),
    ("check ignores duplicates", "bad += seen[i] == seen[i - 1];", "bad += 0;"),
    ("check ignores digests of empty slots", "if (tdig[s] != 0) ++bad;", "if (0) ++bad;"),
    ("check ignores wrong digests", "if (tdig[s] != orc_digest(h)) ++bad;", "if (0) ++bad;"),
    ("interaction without the diagonal", "for (int32_t j = i; j < F; ++j) {",
     "for (int32_t j = i + 1; j < F; ++j) {"),
    ("interaction squares the row", "(double)zb[(int64_t)j * d + k];", "(double)zb[(int64_t)i * d + k];"),
    ("interaction drops the last component", "for (int32_t k = 0; k < d; ++k) {",
     "for (int32_t k = 0; k + 1 < d; ++k) {"),
    ("interaction column-major", "out[o] = acc;",
     "out[b * npairs + (int64_t)j * (j + 1) / 2 + i] = acc;"),
    ("AdaGrad accumulates |g| not g^2", "G[r * ORC_DIM + d] += g * g;",
     "G[r * ORC_DIM + d] += fabs(g);"),
    ("AdaGrad steps against the old accumulator",
     "G[r * ORC_DIM + d] += g * g;\n            w[r * ORC_DIM + d] -= lr * g / (sqrt(G[r * ORC_DIM + d]) + eps);",
     "w[r * ORC_DIM + d] -= lr * g / (sqrt(G[r * ORC_DIM + d]) + eps);\n            G[r * ORC_DIM + d] += g * g;"),
    ("AdaGrad steps up the gradient", "w[r * ORC_DIM + d] -= lr * g", "w[r * ORC_DIM + d] += lr * g"),
    ("sequence gradients dropped", "for (int k = 0; k < 3 && P > 0; ++k) {",
     "for (int k = 0; k < 0 && P > 0; ++k) {"),
    ("sequence rows from the first sub-feature's table", "const int32_t t = seq_table[k];",
     "const int32_t t = seq_table[0];"),
    ("bag gradient from the first table's columns",
     "(double)dpooled[b * (int64_t)T * ORC_DIM + t * ORC_DIM + d];",
     "(double)dpooled[b * (int64_t)T * ORC_DIM + d];"),
    ("a repeated id counted once", "for (int d = 0; d < ORC_DIM; ++d)\n                    grad[r * ORC_DIM + d] +=",
     "for (int d = 0; d < ORC_DIM; ++d)\n                    grad[r * ORC_DIM + d] = "),
    ("backward hash miss not skipped",
     "if (rt < 0 && tables[t].kind == 1) continue;          /* hash miss */",
     "if (0) continue;          /* hash miss */"),
    ("backward resolves every table by floor mod",
     "const int64_t rt = orc_resolve(&tables[t], values[offsets[bag] + i]);",
     "const int64_t rt = orc_floor_mod(values[offsets[bag] + i], tables[t].rows);"),
    ("attention backward: softmax without its mean term", "const double de = p[j] * (dp[j] - pdp);",
     "const double de = p[j] * dp[j];"),
    ("attention backward: ReLU gate of h2 dropped", "dz2[o] = z2[j * 64 + o] > 0.0 ? de * w3[o] : 0.0;",
     "dz2[o] = de * w3[o];"),
    ("attention backward: W2 transposed", "for (int o = 0; o < 64; ++o) a += w2[o * 256 + i] * dz2[o];",
     "for (int o = 0; o < 64; ++o) a += w2[(i % 64) * 256 + (o + 4 * (i / 64))] * dz2[o];"),
    ("attention backward: q*s gradient to q uses q", "gq[b * 48 + c] += dx[c] + dx[96 + c] + sc * dx[144 + c];",
     "gq[b * 48 + c] += dx[c] + dx[96 + c] + q[c] * dx[144 + c];"),
    ("attention backward: q-s sign to s", "dsj[c] += dx[48 + c] - dx[96 + c]", "dsj[c] += dx[48 + c] + dx[96 + c]"),
    ("attention backward: direct term of att dropped", "for (int c = 0; c < 48; ++c) dsj[c] = p[j] * g[c];",
     "for (int c = 0; c < 48; ++c) dsj[c] = 0.0;"),
    ("attention backward: dW1 from h1 not x", "for (int i = 0; i < 192; ++i) dw1[o * 192 + i] += dz1[o] * x[i];",
     "for (int i = 0; i < 192; ++i) dw1[o * 192 + i] += dz1[o] * dz1[i];"),
    ("backward drops the last id of a bag",
     "for (int64_t i = 0; i < lengths[bag]; ++i) {\n                const int64_t rt = orc_resolve(",
     "for (int64_t i = 0; i + 1 < lengths[bag]; ++i) {\n                const int64_t rt = orc_resolve("),
    ("DLRM mean divides by the length + 1", "e[c] /= (double)lengths[bag];",
     "e[c] /= (double)(lengths[bag] + 1);"),
    ("DLRM mean bags summed", "if (modes[t] == 1 && lengths[bag] > 0)", "if (0)"),
    ("DLRM bag drops the last id", "for (int64_t i = 0; i < lengths[bag]; ++i) {\n                const int64_t r = orc_floor_mod(",
     "for (int64_t i = 0; i + 1 < lengths[bag]; ++i) {\n                const int64_t r = orc_floor_mod("),
    ("DLRM bottom reads the first dense row", "orc_dense(wb1, bb1, dense + b * nd, nd, 128, h1);",
     "orc_dense(wb1, bb1, dense, nd, 128, h1);"),
    ("DLRM bottom skips its second layer", "orc_dense(wb2, bb2, h1, 128, d, zb);",
     "for (int32_t c = 0; c < d; ++c) zb[c] = h1[c];"),
    ("DLRM top skips its second layer", "orc_dense(wt2, bt2, t1, 128, 64, t2);",
     "for (int i = 0; i < 64; ++i) t2[i] = t1[i];"),
    ("DLRM logit bias dropped", "double lg = bt3, mag = fabs(bt3);", "double lg = 0.0, mag = fabs(bt3);"),
    ("DLRM sigmoid sign flipped", "prob[b] = 1.0 / (1.0 + exp(-lg));", "prob[b] = 1.0 / (1.0 + exp(lg));"),
    ("DLRM interaction squares the row", "acc += zb[(int64_t)i * d + k] * zb[(int64_t)j * d + k];",
     "acc += zb[(int64_t)i * d + k] * zb[(int64_t)i * d + k];"),
    ("admission above, not at, the threshold", "if (total >= threshold) {", "if (total > threshold) {"),
    ("admission counts an id once per batch", "dc[j] += 1;", "dc[j] = 1;"),
    ("eviction takes the largest score", "if (x->score != y->score) return x->score < y->score ? -1 : 1;",
     "if (x->score != y->score) return x->score > y->score ? -1 : 1;"),
    ("eviction ties take the larger id", "return (x->key > y->key) - (x->key < y->key);",
     "return (x->key < y->key) - (x->key > y->key);"),
    ("eviction scores not saturated", "v[nv].score = tscores[s] < 0xfffffffeull ? tscores[s] : 0xfffffffeull;",
     "v[nv].score = tscores[s];"),
    ("a used id keeps its STEP score", "if (mode == ORC_SCORE_STEP) tscores[s] = step;\n            if (mode == ORC_SCORE_LFU) tscores[s] += dc[j];",
     "if (mode == ORC_SCORE_LFU) tscores[s] += dc[j];"),
    ("an admitted LFU entry starts at 1", "if (mode == ORC_SCORE_LFU) tscores[at] = ctot[q];",
     "if (mode == ORC_SCORE_LFU) tscores[at] = 1;"),
    ("the count survives admission", "if (c >= 0) ccounts[c] = 0;", "if (0) ccounts[c] = 0;"),
    ("admission never reuses a tombstone",
     "while (probes < capacity && tkeys[at] != ORC_EMPTY_KEY && tkeys[at] != ORC_TOMBSTONE) {",
     "while (probes < capacity && tkeys[at] != ORC_EMPTY_KEY) {"),
    ("the tombstone marker counts as an id",
     "if (keys[i] == ORC_EMPTY_KEY || keys[i] == ORC_TOMBSTONE) continue;", "if (keys[i] == ORC_EMPTY_KEY) continue;"),
    ("NO_EVICTION evicts", "if (mode != ORC_SCORE_NONE && ncand > room) {", "if (ncand > room) {"),
    ("left-out candidates lose their counts", "if (c >= 0) ccounts[c] = ctot[q];", "if (c >= 0) ccounts[c] = 0;"),
]


@pytest.mark.parametrize("name,orig,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, orig, repl):
    src = open(oracle.SRC).read()
    # a mistake in a formula goes into every copy of it (the attention's
    # backward recomputes the forward with the same expressions)
    assert src.count(orig) >= 1, f"mutation site not present: {orig!r}"
    msrc = os.path.join(tmp_path, "oracle_mutant.c")
    mlib = os.path.join(tmp_path, "liboracle_mutant.so")
    with open(msrc, "w") as f:
        f.write(src.replace(orig, repl))
    oracle.build(msrc, mlib)
    orc = oracle.Oracle(mlib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant '{name}' passed every pin"

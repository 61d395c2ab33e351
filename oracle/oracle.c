/*
 * CPU oracle for the sparse embedding + DIN attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the forward computes, in fp64.  Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or constant with the HIP library, and the library never calls
 * it.
 *
 * Pages followed (title, section):
 *   [P1] "MultiTowerDIN：当前现状分析"
 *        §2   id features arrive as (values, lengths) and become a
 *             KeyedJaggedTensor
 *        §3   num_buckets: a [N,16] table, row = raw_id % num_buckets
 *        §4.2 DIN attention: cat [q, s, q-s, q*s] on the last dim, attn MLP
 *             (hidden 256, 64), linear to one score, mask + softmax, weighted
 *             sum of the sequence
 *        §4.4 compute graph: pooled deep features; query [B,48]; sequence
 *             [B,100,48]; attn input [B,100,192]; output [B,48]; then the
 *             deep MLP to [B,128], the concat to [B,176] and the final MLP
 *        run-config table: sparse parameters train with AdaGrad (lr 1e-3);
 *        §3   the AdaGrad accumulator is as large as the table
 *   [P2] "MultiTowerDIN：集成 DynamicEmb"
 *        §3.2 lookup is an O(1) open-addressing hash table; an unseen id gives
 *             the constant 0 vector
 *        §4.3 unseen id -> not in the table -> zero embedding
 *        §7   model config: tower hidden units [512, 256, 128], attention MLP
 *             [256, 64], final [64], binary cross entropy loss
 *   [P3] DLRM essay (wmrh.cn/news/12459) §3.2: EmbeddingBag pools each bag
 *        (mode sum)
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - '%' on a negative id is the floor modulo (result in [0, N)), the
 *     semantics of the Python pseudo-code the page prints.
 *   - pooling is a sum; an empty bag pools to 0.
 *   - ReLU after the 256- and 64-wide layers, none after the score layer;
 *     biases on all three layers.
 *   - the mask has -inf semantics: masked positions get weight exactly 0; a
 *     sample with no positions gets output 0.
 *   - only the first max_len positions of a longer sequence are used.
 *   - no softmax temperature or 1/sqrt(d); max-subtracted for range.
 *   - W1 columns: 0-47 q, 48-95 s, 96-143 q-s, 144-191 q*s; inside each block
 *     the sub-features adgroup, cate, brand, 16 each.
 *   - the AdaGrad step is the element-wise one (one accumulator per weight,
 *     starting at 0): G += g^2, w -= lr g / (sqrt(G) + eps), eps 1e-10, no
 *     decay; g is a row's gradient summed over every read of the row in the
 *     batch before the step, and rows the batch does not read are untouched.
 *   - hash lookup: the key is the raw id; a key is present iff some slot holds
 *     it.  The oracle finds it by scanning every slot once (sorted index), so
 *     it depends on no hash function or probe order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_DIM 16
#define ORC_EMPTY_KEY ((int64_t)-1)
#define ORC_TOMBSTONE ((int64_t)-2)      /* a slot whose key was evicted */

/* ---- jagged bookkeeping ([P1] §2: values + lengths -> offsets) ---------- */
void orc_lengths_to_offsets(const int32_t* lengths, int64_t n, int64_t* offsets) {
    offsets[0] = 0;
    for (int64_t i = 0; i < n; ++i) offsets[i + 1] = offsets[i] + (int64_t)lengths[i];
}

/* ---- direct index ([P1] §3: row = raw_id % num_buckets, floor modulo) --- */
int64_t orc_floor_mod(int64_t raw, int64_t n) {
    int64_t r = raw % n;           /* C truncates toward zero: |r| < n */
    if (r < 0) r += n;
    return r;
}

/* ---- hash index ([P2] §3.2, §4.3) ---------------------------------------
 * Scan every slot; collect (key, slot) for occupied slots; sort by key.  A
 * lookup is a binary search in that list: present -> its slot, else -1.     */
typedef struct { int64_t key, slot; } orc_pair;

static int orc_pair_cmp(const void* a, const void* b) {
    int64_t x = ((const orc_pair*)a)->key, y = ((const orc_pair*)b)->key;
    return (x > y) - (x < y);
}

/* Fills sorted_keys/sorted_slots (each of room >= capacity); returns count. */
int64_t orc_hash_index(const int64_t* slot_keys, int64_t capacity,
                       int64_t* sorted_keys, int64_t* sorted_slots) {
    orc_pair* p = (orc_pair*)malloc(sizeof(orc_pair) * (size_t)(capacity > 0 ? capacity : 1));
    int64_t n = 0;
    for (int64_t s = 0; s < capacity; ++s)
        if (slot_keys[s] != ORC_EMPTY_KEY && slot_keys[s] != ORC_TOMBSTONE) { p[n].key = slot_keys[s]; p[n].slot = s; ++n; }
    qsort(p, (size_t)n, sizeof(orc_pair), orc_pair_cmp);
    for (int64_t i = 0; i < n; ++i) { sorted_keys[i] = p[i].key; sorted_slots[i] = p[i].slot; }
    free(p);
    return n;
}

int64_t orc_hash_find(const int64_t* sorted_keys, const int64_t* sorted_slots,
                      int64_t count, int64_t key) {
    int64_t lo = 0, hi = count;               /* search [lo, hi) */
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (sorted_keys[mid] < key) lo = mid + 1; else hi = mid;
    }
    return (lo < count && sorted_keys[lo] == key) ? sorted_slots[lo] : -1;
}

/* ---- hash insert ([P2] §6.4: at start-up the tables are rebuilt by
 * inserting stored key/value pairs; §4.2 score strategies STEP / LFU /
 * NO_EVICTION; §1 slot = key, score, digest, 16 values) ----------------------
 * Placement needs the table convention, a data format: h = SplitMix64's
 * output mix of the key's 64 bits (Steele, Lea & Flood, OOPSLA 2014, with
 * Stafford's "Mix13" shifts and multipliers), home = floor(h * capacity /
 * 2^64), digest = the low byte of h (1 in place of 0, since 0 marks an empty
 * slot), linear probing that wraps, no deletes.  Written here from those
 * definitions, in 128-bit arithmetic.                                       */
static uint64_t orc_mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * UINT64_C(0xbf58476d1ce4e5b9);
    z = (z ^ (z >> 27)) * UINT64_C(0x94d049bb133111eb);
    return z ^ (z >> 31);
}

static int64_t orc_home(uint64_t h, int64_t capacity) {
    __extension__ typedef unsigned __int128 u128;
    return (int64_t)(((u128)h * (u128)(uint64_t)capacity) >> 64);
}

static uint8_t orc_digest(uint64_t h) {
    uint8_t d = (uint8_t)(h & 0xff);
    return d ? d : 1;
}

enum { ORC_SCORE_NONE = 0, ORC_SCORE_STEP = 1, ORC_SCORE_LFU = 2 };

/* Insert-or-assign, one pair after another in the given order.  A key that
 * is stored keeps its slot and takes the new values; a new key takes the
 * first empty slot of its probe sequence (digest and key written); with no
 * empty slot on the whole sequence nothing is stored and its slot is -1
 * (NO_EVICTION: a full table stops accepting keys).  The empty marker is
 * never stored (slot -2).  Scores: STEP writes `step`, LFU adds one (a new
 * slot starts from the empty slot's 0), NONE leaves them.                  */
void orc_hash_insert(int64_t* tkeys, uint8_t* tdig, uint64_t* tscores, float* tvals,
                     int64_t capacity, const int64_t* keys, const float* vals, int64_t n,
                     int32_t mode, uint64_t step, int64_t* slot_out) {
    for (int64_t i = 0; i < n; ++i) {
        const int64_t key = keys[i];
        if (key == ORC_EMPTY_KEY || key == ORC_TOMBSTONE) { slot_out[i] = -2; continue; }
        const uint64_t h = orc_mix64((uint64_t)key);
        int64_t at = orc_home(h, capacity), slot = -1;
        int is_new = 0;
        for (int64_t probes = 0; probes < capacity; ++probes) {
            if (tkeys[at] == key) { slot = at; break; }
            if (tkeys[at] == ORC_EMPTY_KEY) { slot = at; is_new = 1; break; }
            at = (at + 1 == capacity) ? 0 : at + 1;
        }
        slot_out[i] = slot;
        if (slot < 0) continue;
        if (is_new) {
            tkeys[slot] = key;
            tdig[slot] = orc_digest(h);
        }
        memcpy(tvals + slot * ORC_DIM, vals + i * ORC_DIM, sizeof(float) * ORC_DIM);
        if (mode == ORC_SCORE_STEP) tscores[slot] = step;
        if (mode == ORC_SCORE_LFU) tscores[slot] = tscores[slot] + 1;
    }
}

static int orc_i64_cmp(const void* a, const void* b) {
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x > y) - (x < y);
}

/* Slots that break the convention: an empty slot with a nonzero digest, a
 * stored key with the wrong digest, a stored key with an empty slot between
 * its home and its slot (a lookup would miss it), or a key stored twice.    */
int64_t orc_hash_check(const int64_t* tkeys, const uint8_t* tdig, int64_t capacity) {
    int64_t bad = 0, n = 0;
    int64_t* seen = (int64_t*)malloc(sizeof(int64_t) * (size_t)(capacity > 0 ? capacity : 1));
    for (int64_t s = 0; s < capacity; ++s) {
        if (tkeys[s] == ORC_EMPTY_KEY) {
            if (tdig[s] != 0) ++bad;
            continue;
        }
        if (tkeys[s] == ORC_TOMBSTONE) {        /* a deleted key: probes pass it */
            if (tdig[s] == 0) ++bad;
            continue;
        }
        seen[n++] = tkeys[s];
        const uint64_t h = orc_mix64((uint64_t)tkeys[s]);
        if (tdig[s] != orc_digest(h)) ++bad;
        for (int64_t q = orc_home(h, capacity); q != s; q = (q + 1 == capacity) ? 0 : q + 1)
            if (tkeys[q] == ORC_EMPTY_KEY) { ++bad; break; }
    }
    qsort(seen, (size_t)n, sizeof(int64_t), orc_i64_cmp);
    for (int64_t i = 1; i < n; ++i) bad += seen[i] == seen[i - 1];
    free(seen);
    return bad;
}

/* ---- DLRM dot-product interaction ([P3] DLRM essay §2.3, §3.1, §4.2: the
 * interaction layer takes, per sample, the bottom MLP's output and every
 * pooled embedding, F vectors of width d, and emits the dot product of every
 * pair i <= j -- the upper triangle with the diagonal, as the essay's loop runs
 * j from i -- row by row: (0,0), (0,1), ..., (0,F-1), (1,1), ...) ----------
 * z [B][F][d]; out [B][F(F+1)/2]; scale (or NULL) gets sum_k |z_ik z_jk|,
 * the size of each dot product's terms.                                    */
void orc_dlrm_interact(const float* z, int64_t B, int32_t F, int32_t d, double* out, double* scale) {
    const int64_t npairs = (int64_t)F * (F + 1) / 2;
    for (int64_t b = 0; b < B; ++b) {
        const float* zb = z + b * F * d;
        int64_t o = b * npairs;
        for (int32_t i = 0; i < F; ++i) {
            for (int32_t j = i; j < F; ++j) {
                double acc = 0.0, mag = 0.0;
                for (int32_t k = 0; k < d; ++k) {
                    const double t = (double)zb[(int64_t)i * d + k] * (double)zb[(int64_t)j * d + k];
                    acc += t;
                    mag += fabs(t);
                }
                out[o] = acc;
                if (scale) scale[o] = mag;
                ++o;
            }
        }
    }
}

/* One table as the oracle sees it. */
typedef struct {
    int32_t kind;                 /* 0 direct, 1 hash */
    int32_t pad_;
    int64_t rows;                 /* direct: num_buckets; hash: capacity */
    const float* values;          /* [rows][16] */
    const int64_t* sorted_keys;   /* hash: index built by orc_hash_index */
    const int64_t* sorted_slots;
    int64_t count;
} orc_table;

/* Row of a raw id in a table: direct -> floor mod; hash -> slot or -1. */
int64_t orc_resolve(const orc_table* t, int64_t raw) {
    if (t->kind == 0) return orc_floor_mod(raw, t->rows);
    return orc_hash_find(t->sorted_keys, t->sorted_slots, t->count, raw);
}

void orc_resolve_many(const orc_table* t, const int64_t* raw, int64_t n, int64_t* rows) {
    for (int64_t i = 0; i < n; ++i) rows[i] = orc_resolve(t, raw[i]);
}

/* ---- sparse backward of the bags + AdaGrad step ([P1] run-config table:
 * sparse parameters train with AdaGrad, lr 1e-3; [P1] §3: the AdaGrad
 * accumulator is as large as the table, one value per weight; [P2] §3.3:
 * the gradient is accumulated in fp32 or wider) -------------------------------
 * All T tables sit in one flat row space: table t owns rows base[t] ..
 * base[t] + tables[t].rows - 1 of w, G, grad and touched ([R][16] / [R]); a
 * hash table's rows are its slots.
 * The gradient of a weight row is the sum of the output gradients of every
 * place that row was read:
 *   - each id of bag (t, b) adds dpooled[b][16t .. 16t+16) to the row of the
 *     id in table t (direct: floor_mod(id, rows); hash: the slot holding the
 *     id) -- the pooled sum reads it once per id, so a repeated id adds its
 *     bag's gradient once per repetition.  A hash miss reads the constant zero
 *     vector ([P2] §3.2), no row: its gradient goes nowhere;
 *   - each packed sequence position j < P of sub-feature k adds
 *     dseq[k][j][0..16) to the row of seq_values[k*seq_stride + j] in table
 *     seq_table[k] (the unpooled sequence rows the attention reads).
 * grad receives that sum (it must be zero on entry) and touched marks each row
 * read at least once.  Then every touched row takes one element-wise AdaGrad
 * step with its summed gradient g:
 *   G += g * g;   w -= lr * g / (sqrt(G) + eps).
 * Untouched rows are left as they are.  Returns the number of reads whose
 * row fell outside its table (0 unless the row arithmetic is broken); those
 * are skipped, never written.                                              */
int64_t orc_embbag_adagrad(int32_t T, int64_t B, const orc_table* tables, const int64_t* base,
                        const int64_t* values, const int32_t* lengths, const int64_t* offsets,
                        const float* dpooled, int64_t P, const int32_t* seq_table,
                        const int64_t* seq_values, int64_t seq_stride, const float* dseq,
                        double lr, double eps, double* w, double* G, double* grad,
                        uint8_t* touched) {
    int64_t outside = 0;
    for (int32_t t = 0; t < T; ++t) {
        for (int64_t b = 0; b < B; ++b) {
            const int64_t bag = (int64_t)t * B + b;
            for (int64_t i = 0; i < lengths[bag]; ++i) {
                const int64_t rt = orc_resolve(&tables[t], values[offsets[bag] + i]);
                if (rt < 0 && tables[t].kind == 1) continue;          /* hash miss */
                if (rt < 0 || rt >= tables[t].rows) { ++outside; continue; }
                const int64_t r = base[t] + rt;
                touched[r] = 1;
                for (int d = 0; d < ORC_DIM; ++d)
                    grad[r * ORC_DIM + d] += (double)dpooled[b * (int64_t)T * ORC_DIM + t * ORC_DIM + d];
            }
        }
    }
    for (int k = 0; k < 3 && P > 0; ++k) {
        const int32_t t = seq_table[k];
        for (int64_t j = 0; j < P; ++j) {
            const int64_t rt = orc_resolve(&tables[t], seq_values[k * seq_stride + j]);
            if (rt < 0 && tables[t].kind == 1) continue;              /* hash miss */
            if (rt < 0 || rt >= tables[t].rows) { ++outside; continue; }
            const int64_t r = base[t] + rt;
            touched[r] = 1;
            for (int d = 0; d < ORC_DIM; ++d)
                grad[r * ORC_DIM + d] += (double)dseq[(k * P + j) * ORC_DIM + d];
        }
    }
    const int64_t R = base[T - 1] + tables[T - 1].rows;
    for (int64_t r = 0; r < R; ++r) {
        if (!touched[r]) continue;
        for (int d = 0; d < ORC_DIM; ++d) {
            const double g = grad[r * ORC_DIM + d];
            G[r * ORC_DIM + d] += g * g;
            w[r * ORC_DIM + d] -= lr * g / (sqrt(G[r * ORC_DIM + d]) + eps);
        }
    }
    return outside;
}

/* Embedding of a raw id: the table row, or the zero vector on a hash miss. */
static void orc_emb(const orc_table* t, int64_t raw, double* out16) {
    int64_t r = orc_resolve(t, raw);
    for (int d = 0; d < ORC_DIM; ++d) out16[d] = r < 0 ? 0.0 : (double)t->values[r * ORC_DIM + d];
}

/* ---- sum-pooled embedding bags ([P1] §3, §4.4; [P3] §3.2) ---------------
 * pooled[s][16k + d] = sum over the ids of bag (k, b) of table k's row[d],
 * for b = samples[s]; bag (k, b) is values[offsets[k*B+b] .. + lengths[k*B+b]).
 * An empty bag pools to 0.                                                  */
void orc_embbag(int32_t T, int64_t B, const orc_table* tables,
                const int64_t* values, const int32_t* lengths, const int64_t* offsets,
                const int64_t* samples, int64_t ns, double* pooled) {
    for (int64_t s = 0; s < ns; ++s) {
        int64_t b = samples[s];
        for (int32_t k = 0; k < T; ++k) {
            int64_t bag = (int64_t)k * B + b;
            double acc[ORC_DIM];
            for (int d = 0; d < ORC_DIM; ++d) acc[d] = 0.0;
            for (int64_t i = 0; i < lengths[bag]; ++i) {
                int64_t r = orc_resolve(&tables[k], values[offsets[bag] + i]);
                if (r < 0) continue;                 /* hash miss: the zero vector */
                for (int d = 0; d < ORC_DIM; ++d) acc[d] += (double)tables[k].values[r * ORC_DIM + d];
            }
            for (int d = 0; d < ORC_DIM; ++d) pooled[s * (int64_t)T * ORC_DIM + k * ORC_DIM + d] = acc[d];
        }
    }
}

/* ---- DIN target attention ([P1] §4.2, §4.4) -----------------------------
 * For sample b = samples[s], with L = min(seq_lengths[b], max_len):
 *   s_j   = rows of the three sub-features at position j (48 values)
 *   x_j   = [q, s_j, q - s_j, q * s_j]                    (192)
 *   h1    = relu(W1 x_j + b1)   W1 [256][192]
 *   h2    = relu(W2 h1 + b2)    W2 [64][256]
 *   e_j   = w3 . h2 + b3
 *   p_j   = exp(e_j - max e) / sum_k exp(e_k - max e)
 *   att   = sum_j p_j s_j                                  (48)
 * L = 0 gives att = 0.  query[s] is sample b's 48-value query.
 * scores / weights (optional, [ns][max_len]) receive e_j and p_j.          */
void orc_din(const orc_table* seq_tables /* 3: adgroup, cate, brand */,
             const int64_t* seq_values, int64_t seq_stride,
             const int64_t* seq_offsets, const int32_t* seq_lengths, int32_t max_len,
             const double* query,
             const double* w1, const double* b1, const double* w2, const double* b2,
             const double* w3, double b3,
             const int64_t* samples, int64_t ns,
             double* att, double* scores, double* weights) {
    double* sj = (double*)malloc(sizeof(double) * 48 * (size_t)(max_len > 0 ? max_len : 1));
    double* e = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    double x[192], h1[256], h2[64];
    for (int64_t s = 0; s < ns; ++s) {
        int64_t b = samples[s];
        int64_t L = seq_lengths[b] < max_len ? seq_lengths[b] : max_len;
        const double* q = query + s * 48;
        double* out = att + s * 48;
        if (scores) for (int j = 0; j < max_len; ++j) scores[s * max_len + j] = 0.0;
        if (weights) for (int j = 0; j < max_len; ++j) weights[s * max_len + j] = 0.0;
        if (L <= 0) { for (int c = 0; c < 48; ++c) out[c] = 0.0; continue; }
        for (int64_t j = 0; j < L; ++j) {
            for (int f = 0; f < 3; ++f) {
                int64_t raw = seq_values[f * seq_stride + seq_offsets[b] + j];
                orc_emb(&seq_tables[f], raw, sj + j * 48 + f * 16);
            }
            for (int c = 0; c < 48; ++c) {
                double qc = q[c], sc = sj[j * 48 + c];
                x[c] = qc;
                x[48 + c] = sc;
                x[96 + c] = qc - sc;
                x[144 + c] = qc * sc;
            }
            for (int o = 0; o < 256; ++o) {
                double a = b1[o];
                for (int i = 0; i < 192; ++i) a += w1[o * 192 + i] * x[i];
                h1[o] = a > 0.0 ? a : 0.0;
            }
            for (int o = 0; o < 64; ++o) {
                double a = b2[o];
                for (int i = 0; i < 256; ++i) a += w2[o * 256 + i] * h1[i];
                h2[o] = a > 0.0 ? a : 0.0;
            }
            double a = b3;
            for (int i = 0; i < 64; ++i) a += w3[i] * h2[i];
            e[j] = a;
        }
        double m = e[0];
        for (int64_t j = 1; j < L; ++j) if (e[j] > m) m = e[j];
        double den = 0.0;
        for (int64_t j = 0; j < L; ++j) den += exp(e[j] - m);
        for (int c = 0; c < 48; ++c) out[c] = 0.0;
        for (int64_t j = 0; j < L; ++j) {
            double p = exp(e[j] - m) / den;
            for (int c = 0; c < 48; ++c) out[c] += p * sj[j * 48 + c];
            if (scores) scores[s * max_len + j] = e[j];
            if (weights) weights[s * max_len + j] = p;
        }
    }
    free(sj);
    free(e);
}

/* ---- DIN attention backward (the training step of [P1]'s run-config table
 * through the attention of [P1] §4.2 / §4.4) --------------------------------
 * For every sample b with L = min(seq_lengths[b], max_len) positions and the
 * gradient g = gatt[b] (48) of its attention output, the forward is
 * recomputed (s_j, x_j = [q, s_j, q - s_j, q * s_j], z1_j = W1 x_j + b1,
 * h1_j = relu(z1_j), z2_j = W2 h1_j + b2, h2_j = relu(z2_j),
 * e_j = w3 . h2_j + b3, p_j = softmax(e)_j) and differentiated by the chain
 * rule, in the order of that forward read backwards:
 *   att = sum_j p_j s_j:      dp_j = g . s_j,   ds_j = p_j g
 *   softmax:                  de_j = p_j (dp_j - sum_k p_k dp_k)
 *   e_j = w3 . h2_j + b3:     dw3 += de_j h2_j,  db3 += de_j,  dh2_j = de_j w3
 *   h2_j = relu(z2_j):        dz2_j = dh2_j where z2_j > 0, else 0
 *   z2_j = W2 h1_j + b2:      dW2 += dz2_j h1_j^T,  db2 += dz2_j,  dh1_j = W2^T dz2_j
 *   h1_j = relu(z1_j):        dz1_j = dh1_j where z1_j > 0, else 0
 *   z1_j = W1 x_j + b1:       dW1 += dz1_j x_j^T,  db1 += dz1_j,  dx_j = W1^T dz1_j
 *   x_j = [q, s, q-s, q*s]:   dq += dx[0:48] + dx[96:144] + s_j * dx[144:192]
 *                             ds_j += dx[48:96] - dx[96:144] + q * dx[144:192]
 * A sample with no positions has att = 0 for every q: it contributes nothing.
 * gq [B][48]; gs [seq_stride][48] by position index seq_offsets[b] + j (zero
 * for positions past max_len); the weight gradients are sums over all
 * samples and positions (they must be zero on entry).  db3 is zero in exact
 * arithmetic (every score moving by the same amount leaves the softmax
 * unchanged), so db3_scale receives sum |de_j|, the size of its terms, the
 * yardstick for its rounding; likewise gq, whose terms of a sample nearly
 * cancel when its positions look alike (de_j is a difference of nearly equal
 * terms and the de_j sum to zero), gets gq_scale [B][48]: the chain above run
 * on the sizes of the terms instead of their values (a running-error bound
 * of the kind Higham, "Accuracy and Stability of Numerical Algorithms", §3,
 * uses for sums and products).  The ReLU gates of the chain (z > 0) are
 * decided in fp64; a z within a few roundings of zero may fall the other way
 * in a lower precision, and the derivative of ReLU at 0 is not fixed by the
 * method, so either decision is valid there.  For checking such units, gate
 * (or NULL) receives per position index [seq_stride][576]: z1_j / a1_j
 * (256; a1_j = |b1| + sum_i |W1[u][i] x_j[i]|, the size of z1's terms), dh1_j
 * = W2^T dz2_j before its gate (256), and z2_j / a2_j (64, a2_j likewise).
 * Returns nothing. */
void orc_din_bwd(const orc_table* seq_tables, const int64_t* seq_values, int64_t seq_stride,
                 const int64_t* seq_offsets, const int32_t* seq_lengths, int32_t max_len,
                 int64_t B, const double* query, const double* w1, const double* b1,
                 const double* w2, const double* b2, const double* w3, double b3,
                 const double* gatt, double* gq, double* gs, double* dw1, double* db1,
                 double* dw2, double* db2, double* dw3, double* db3, double* db3_scale,
                 double* gq_scale, double* gate) {
    const int64_t ml = max_len > 0 ? max_len : 1;
    double* sj = (double*)malloc(sizeof(double) * 48 * (size_t)ml);
    double* xs = (double*)malloc(sizeof(double) * 192 * (size_t)ml);
    double* z1 = (double*)malloc(sizeof(double) * 256 * (size_t)ml);
    double* z2 = (double*)malloc(sizeof(double) * 64 * (size_t)ml);
    double* e = (double*)malloc(sizeof(double) * (size_t)ml);
    double* p = (double*)malloc(sizeof(double) * (size_t)ml);
    double* dp = (double*)malloc(sizeof(double) * (size_t)ml);
    for (int64_t i = 0; i < seq_stride * 48; ++i) gs[i] = 0.0;
    if (gate)
        for (int64_t i = 0; i < seq_stride * 576; ++i) gate[i] = 0.0;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t L = seq_lengths[b] < max_len ? seq_lengths[b] : max_len;
        const double* q = query + b * 48;
        const double* g = gatt + b * 48;
        for (int c = 0; c < 48; ++c) gq[b * 48 + c] = gq_scale[b * 48 + c] = 0.0;
        if (L <= 0) continue;
        /* forward, kept per position */
        for (int64_t j = 0; j < L; ++j) {
            for (int f = 0; f < 3; ++f)
                orc_emb(&seq_tables[f], seq_values[f * seq_stride + seq_offsets[b] + j],
                        sj + j * 48 + f * 16);
            double* x = xs + j * 192;
            for (int c = 0; c < 48; ++c) {
                const double qc = q[c], sc = sj[j * 48 + c];
                x[c] = qc;
                x[48 + c] = sc;
                x[96 + c] = qc - sc;
                x[144 + c] = qc * sc;
            }
            for (int o = 0; o < 256; ++o) {
                double a = b1[o];
                for (int i = 0; i < 192; ++i) a += w1[o * 192 + i] * x[i];
                z1[j * 256 + o] = a;
            }
            for (int o = 0; o < 64; ++o) {
                double a = b2[o];
                for (int i = 0; i < 256; ++i) a += w2[o * 256 + i] * (z1[j * 256 + i] > 0.0 ? z1[j * 256 + i] : 0.0);
                z2[j * 64 + o] = a;
            }
            double a = b3;
            for (int i = 0; i < 64; ++i) a += w3[i] * (z2[j * 64 + i] > 0.0 ? z2[j * 64 + i] : 0.0);
            e[j] = a;
        }
        double m = e[0];
        for (int64_t j = 1; j < L; ++j) if (e[j] > m) m = e[j];
        double den = 0.0;
        for (int64_t j = 0; j < L; ++j) den += exp(e[j] - m);
        for (int64_t j = 0; j < L; ++j) p[j] = exp(e[j] - m) / den;
        /* att = sum_j p_j s_j */
        double pdp = 0.0, pdp_mag = 0.0;
        for (int64_t j = 0; j < L; ++j) {
            double d = 0.0;
            for (int c = 0; c < 48; ++c) d += g[c] * sj[j * 48 + c];
            dp[j] = d;
            pdp += p[j] * d;
            pdp_mag += p[j] * fabs(d);
        }
        for (int64_t j = 0; j < L; ++j) {
            double* dsj = gs + (seq_offsets[b] + j) * 48;
            for (int c = 0; c < 48; ++c) dsj[c] = p[j] * g[c];
            const double de = p[j] * (dp[j] - pdp);                 /* softmax */
            double dz2[64], dz1[256], dx[192];
            *db3 += de;
            *db3_scale += fabs(de);
            for (int o = 0; o < 64; ++o) {
                const double h2o = z2[j * 64 + o] > 0.0 ? z2[j * 64 + o] : 0.0;
                dw3[o] += de * h2o;
                dz2[o] = z2[j * 64 + o] > 0.0 ? de * w3[o] : 0.0;
            }
            for (int o = 0; o < 64; ++o) {
                db2[o] += dz2[o];
                for (int i = 0; i < 256; ++i)
                    dw2[o * 256 + i] += dz2[o] * (z1[j * 256 + i] > 0.0 ? z1[j * 256 + i] : 0.0);
            }
            double* gt = gate ? gate + (seq_offsets[b] + j) * 576 : NULL;
            for (int i = 0; i < 256; ++i) {
                double a = 0.0;
                for (int o = 0; o < 64; ++o) a += w2[o * 256 + i] * dz2[o];
                dz1[i] = z1[j * 256 + i] > 0.0 ? a : 0.0;
                if (gt) gt[256 + i] = a;
            }
            const double* x = xs + j * 192;
            if (gt) {
                for (int o = 0; o < 256; ++o) {
                    double a1 = fabs(b1[o]);
                    for (int i = 0; i < 192; ++i) a1 += fabs(w1[o * 192 + i] * x[i]);
                    gt[o] = a1 > 0.0 ? z1[j * 256 + o] / a1 : 0.0;
                }
                for (int o = 0; o < 64; ++o) {
                    double a2 = fabs(b2[o]);
                    for (int i = 0; i < 256; ++i)
                        a2 += fabs(w2[o * 256 + i] * (z1[j * 256 + i] > 0.0 ? z1[j * 256 + i] : 0.0));
                    gt[512 + o] = a2 > 0.0 ? z2[j * 64 + o] / a2 : 0.0;
                }
            }
            for (int o = 0; o < 256; ++o) {
                db1[o] += dz1[o];
                for (int i = 0; i < 192; ++i) dw1[o * 192 + i] += dz1[o] * x[i];
            }
            for (int i = 0; i < 192; ++i) {
                double a = 0.0;
                for (int o = 0; o < 256; ++o) a += w1[o * 192 + i] * dz1[o];
                dx[i] = a;
            }
            /* the same chain on the sizes of the terms (|de_j|'s terms, then
             * |w3|, |W2|^T, |W1|^T under the same ReLU gates): the yardstick of
             * gq, whose terms nearly cancel when a sample's positions look alike */
            double m2[64], m1[256], mx[192];
            const double de_mag = p[j] * (fabs(dp[j]) + pdp_mag);
            for (int o = 0; o < 64; ++o) m2[o] = z2[j * 64 + o] > 0.0 ? de_mag * fabs(w3[o]) : 0.0;
            for (int i = 0; i < 256; ++i) {
                double a = 0.0;
                for (int o = 0; o < 64; ++o) a += fabs(w2[o * 256 + i]) * m2[o];
                m1[i] = z1[j * 256 + i] > 0.0 ? a : 0.0;
            }
            for (int i = 0; i < 192; ++i) {
                double a = 0.0;
                for (int o = 0; o < 256; ++o) a += fabs(w1[o * 192 + i]) * m1[o];
                mx[i] = a;
            }
            for (int c = 0; c < 48; ++c) {
                const double sc = sj[j * 48 + c];
                gq[b * 48 + c] += dx[c] + dx[96 + c] + sc * dx[144 + c];
                gq_scale[b * 48 + c] += mx[c] + mx[96 + c] + fabs(sc) * mx[144 + c];
                dsj[c] += dx[48 + c] - dx[96 + c] + q[c] * dx[144 + c];
            }
        }
    }
    free(sj); free(xs); free(z1); free(z2); free(e); free(p); free(dp);
}

/* ------------------------------------------------------------------------
 * Deep tower and final MLP: the rest of the MultiTowerDIN forward
 * ([P1] §4.4 compute graph: the deep MLP 512 -> 256 -> 128 on the pooled deep
 * features, the concat of its [B,128] output with the [B,48] attention
 * output into [B,176], the final MLP 176 -> 64 -> 1; [P2] §7 model config:
 * tower hidden units [512, 256, 128], final hidden units [64]; the loss is
 * binary cross entropy, so the last unit is a logit).
 *   d1    = relu(Wd1 x  + bd1)    Wd1 [512][256], x = pooled deep row (256)
 *   d2    = relu(Wd2 d1 + bd2)    Wd2 [256][512]
 *   d3    = relu(Wd3 d2 + bd3)    Wd3 [128][256]      -> deep_out
 *   z     = [d3, att]                                 (176)
 *   f     = relu(Wf z + bf)       Wf  [64][176]
 *   logit = wo . f + bo;  prob = 1 / (1 + exp(-logit))
 * Readings: ReLU after every hidden layer, none on the logit; biases on every
 * layer; the deep output comes first in the concat (the page's order).
 * pooled has row stride `ld` (>= 256); att is [ns][48]; deep_out [ns][128],
 * logit [ns] and prob [ns] (deep_out and prob may be NULL).  lscale [ns]
 * (or NULL) receives |bo| + sum_i |wo_i f_i|, the size of the logit's terms:
 * the yardstick for the error of a logit that cancels to near zero.       */
static void orc_layer(const double* W, const double* bias, const double* in, int nin,
                      int nout, double* out) {
    for (int o = 0; o < nout; ++o) {
        double acc = bias[o];
        for (int i = 0; i < nin; ++i) acc += W[(int64_t)o * nin + i] * in[i];
        out[o] = acc > 0.0 ? acc : 0.0;
    }
}

void orc_towers(int64_t ns, const double* pooled, int64_t ld, const double* att,
                const double* wd1, const double* bd1, const double* wd2, const double* bd2,
                const double* wd3, const double* bd3, const double* wf, const double* bf,
                const double* wo, double bo,
                double* deep_out, double* logit, double* prob, double* lscale) {
    double d1[512], d2[256], z[176], f[64];
    for (int64_t s = 0; s < ns; ++s) {
        orc_layer(wd1, bd1, pooled + s * ld, 256, 512, d1);
        orc_layer(wd2, bd2, d1, 512, 256, d2);
        orc_layer(wd3, bd3, d2, 256, 128, z);
        for (int c = 0; c < 48; ++c) z[128 + c] = att[s * 48 + c];
        orc_layer(wf, bf, z, 176, 64, f);
        double lg = bo, mag = fabs(bo);
        for (int i = 0; i < 64; ++i) {
            lg += wo[i] * f[i];
            mag += fabs(wo[i] * f[i]);
        }
        if (lscale) lscale[s] = mag;
        if (deep_out) for (int c = 0; c < 128; ++c) deep_out[s * 128 + c] = z[c];
        logit[s] = lg;
        if (prob) prob[s] = 1.0 / (1.0 + exp(-lg));
    }
}

/* ------------------------------------------------------------------------
 * DLRM forward ([P3] §2.3: four layers with separate duties -- a bottom MLP
 * maps the dense features to a vector of the embedding width, per-table
 * EmbeddingBags pool the sparse ids, the interaction layer takes the dot
 * product of every pair of those vectors (upper triangle only), a top MLP
 * turns the dot products into the prediction; §3.2: a bag pools by sum or by
 * mean; §3.3 and §4.2: with S sparse features and one dense vector the
 * interaction has (S+1)(S+2)/2 outputs, the pairs (i, j) with j running from
 * i, and the top MLP takes exactly those; §4.2's layer widths: bottom
 * n_dense -> 128 -> d with ReLU after both layers, top -> 128 -> 64 -> 1 with
 * ReLU, ReLU, sigmoid).
 *   h   = relu(Wb2 relu(Wb1 x + bb1) + bb2)            x = dense row (n_dense)
 *   e_t = sum (or mean) over bag (t, b) of table t's rows (d each); an
 *         empty bag gives 0 in both modes
 *   z   = [h, e_0, ..., e_{S-1}]                       (S+1 vectors of width d)
 *   I   = <z_i, z_j> for i <= j, row order (0,0), (0,1), ..., (S,S)
 *   t1  = relu(Wt1 I + bt1);  t2 = relu(Wt2 t1 + bt2)
 *   logit = wt3 . t2 + bt3;   prob = 1 / (1 + exp(-logit))
 * Readings: the tables are direct (row = floor_mod(id, rows)); the bags are
 * the key-major KJT (bag t*B + b holds values[offsets[bag] .. + lengths[bag]));
 * biases on every layer.  tables[t] points at table t's [rows[t]][d] fp32
 * rows; modes[t] is 0 for sum, 1 for mean.  Outputs: z [B][S+1][d], inter
 * [B][npairs], logit [B], prob [B]; lscale [B] (or NULL) receives |bt3| +
 * sum_i |wt3_i t2_i|, the size of the logit's terms; iscale [B][npairs] (or
 * NULL) receives sum_k |z_ik z_jk|.                                        */
static void orc_dense(const double* W, const double* bias, const double* in, int nin, int nout,
                      double* out) {
    for (int o = 0; o < nout; ++o) {
        double acc = bias[o];
        for (int i = 0; i < nin; ++i) acc += W[(int64_t)o * nin + i] * in[i];
        out[o] = acc > 0.0 ? acc : 0.0;
    }
}

void orc_dlrm_fwd(int64_t B, int32_t nd, int32_t d, int32_t S, const double* dense,
                  const double* wb1, const double* bb1, const double* wb2, const double* bb2,
                  const int64_t* rows, const float* const* tables, const int32_t* modes,
                  const int64_t* values, const int32_t* lengths, const int64_t* offsets,
                  const double* wt1, const double* bt1, const double* wt2, const double* bt2,
                  const double* wt3, double bt3, double* z, double* inter, double* logit,
                  double* prob, double* lscale, double* iscale) {
    const int32_t F = S + 1;
    const int64_t npairs = (int64_t)F * (F + 1) / 2;
    double h1[128], t1[128], t2[64];
    for (int64_t b = 0; b < B; ++b) {
        double* zb = z + b * F * d;
        orc_dense(wb1, bb1, dense + b * nd, nd, 128, h1);
        orc_dense(wb2, bb2, h1, 128, d, zb);
        for (int32_t t = 0; t < S; ++t) {
            double* e = zb + (int64_t)(1 + t) * d;
            for (int32_t c = 0; c < d; ++c) e[c] = 0.0;
            const int64_t bag = (int64_t)t * B + b;
            for (int64_t i = 0; i < lengths[bag]; ++i) {
                const int64_t r = orc_floor_mod(values[offsets[bag] + i], rows[t]);
                for (int32_t c = 0; c < d; ++c) e[c] += (double)tables[t][r * d + c];
            }
            if (modes[t] == 1 && lengths[bag] > 0)
                for (int32_t c = 0; c < d; ++c) e[c] /= (double)lengths[bag];
        }
        double* ib = inter + b * npairs;
        int64_t o = 0;
        for (int32_t i = 0; i < F; ++i)
            for (int32_t j = i; j < F; ++j) {
                double acc = 0.0, mag = 0.0;
                for (int32_t k = 0; k < d; ++k) {
                    acc += zb[(int64_t)i * d + k] * zb[(int64_t)j * d + k];
                    mag += fabs(zb[(int64_t)i * d + k] * zb[(int64_t)j * d + k]);
                }
                ib[o] = acc;
                if (iscale) iscale[b * npairs + o] = mag;
                ++o;
            }
        orc_dense(wt1, bt1, ib, (int)npairs, 128, t1);
        orc_dense(wt2, bt2, t1, 128, 64, t2);
        double lg = bt3, mag = fabs(bt3);
        for (int i = 0; i < 64; ++i) {
            lg += wt3[i] * t2[i];
            mag += fabs(wt3[i] * t2[i]);
        }
        logit[b] = lg;
        prob[b] = 1.0 / (1.0 + exp(-lg));
        if (lscale) lscale[b] = mag;
    }
}

/* ------------------------------------------------------------------------
 * Frequency admission and score-driven eviction, one batch of ids at a time
 * ([P2] §4.1: an id enters its table only once it has been seen at least
 * `threshold` times, and until then reads the constant 0 vector; §4.2: the
 * score strategy picks what leaves a full table -- STEP the entry inserted
 * earliest, LFU the one used least, NO_EVICTION none, so a full table stops
 * taking ids; §2 and §7: an initializer gives a new row its values).
 * Readings (the pages give no algorithm):
 *   - the ids of a call are taken together: each distinct id counts once per
 *     occurrence; the distinct ids are processed in the order of their first
 *     occurrence;
 *   - an id already stored is "used": STEP sets its score to `step`, LFU
 *     adds its number of occurrences, NO_EVICTION leaves scores alone;
 *   - an id not stored adds its occurrences to its count in the counter
 *     table (a second key -> count table, 0 when absent); it becomes a
 *     candidate when the count reaches `threshold`, else the count is kept;
 *   - the table holds at most max_keys ids.  Candidates are admitted in
 *     first-occurrence order while there is room; for the rest, STEP and LFU
 *     first evict as many entries stored before the call as there are
 *     candidates left, the smallest scores first (scores compared after
 *     saturating at 2^32 - 2; equal scores: the smaller id first, so the
 *     choice does not depend on where ids were placed), and then
 *     admit that many more; candidates still left keep their counts;
 *   - an evicted slot becomes a tombstone (key -2, digest kept, score 0):
 *     lookups pass it, inserts may reuse it; -1 and -2 are never stored;
 *   - an admitted id takes the first empty or tombstone slot of its probe
 *     sequence, its digest, init_vals of its first occurrence, the score
 *     `step` (STEP), its count (LFU) or none (NO_EVICTION); its count in the
 *     counter table becomes 0;
 *   - a new id whose count has no room in a full counter table is not
 *     counted (its count stays 0 before this call's occurrences).
 * slot_out[i] is the slot holding keys[i] after the call, -1 if absent, -2
 * for the reserved keys.  counts_out (3): ids admitted, entries evicted,
 * candidates left out.  The tables are searched by scanning their slots, so
 * nothing here depends on probe order except where a new id is placed.     */
static int64_t orc_scan_find(const int64_t* k, int64_t cap, int64_t key) {
    for (int64_t s = 0; s < cap; ++s)
        if (k[s] == key) return s;
    return -1;
}

typedef struct { uint64_t score; int64_t key, slot; } orc_victim;

static int orc_victim_cmp(const void* a, const void* b) {
    const orc_victim* x = (const orc_victim*)a;
    const orc_victim* y = (const orc_victim*)b;
    if (x->score != y->score) return x->score < y->score ? -1 : 1;
    return (x->key > y->key) - (x->key < y->key);
}

void orc_hash_admit(int64_t* tkeys, uint8_t* tdig, uint64_t* tscores, float* tvals,
                    int64_t capacity, int64_t max_keys, int64_t* ckeys, uint64_t* ccounts,
                    int64_t ccap, const int64_t* keys, const float* init_vals, int64_t n,
                    uint64_t threshold, int32_t mode, uint64_t step, int64_t* slot_out,
                    int64_t* counts_out) {
    int64_t* dk = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));   /* distinct ids */
    int64_t* df = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));   /* first index */
    uint64_t* dc = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)(n > 0 ? n : 1)); /* occurrences */
    int64_t nd = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (keys[i] == ORC_EMPTY_KEY || keys[i] == ORC_TOMBSTONE) continue;
        int64_t j = 0;
        while (j < nd && dk[j] != keys[i]) ++j;
        if (j == nd) { dk[nd] = keys[i]; df[nd] = i; dc[nd] = 0; ++nd; }
        dc[j] += 1;
    }
    int64_t stored = 0;
    for (int64_t s = 0; s < capacity; ++s)
        stored += tkeys[s] != ORC_EMPTY_KEY && tkeys[s] != ORC_TOMBSTONE;
    int64_t* cand = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nd > 0 ? nd : 1));
    uint64_t* ctot = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)(nd > 0 ? nd : 1));
    int64_t ncand = 0;
    for (int64_t j = 0; j < nd; ++j) {
        const int64_t s = orc_scan_find(tkeys, capacity, dk[j]);
        if (s >= 0) {
            if (mode == ORC_SCORE_STEP) tscores[s] = step;
            if (mode == ORC_SCORE_LFU) tscores[s] += dc[j];
            continue;
        }
        const int64_t c = orc_scan_find(ckeys, ccap, dk[j]);
        const uint64_t total = (c >= 0 ? ccounts[c] : 0) + dc[j];
        if (total >= threshold) {
            cand[ncand] = j;
            ctot[ncand] = total;
            ++ncand;
        } else if (c >= 0) {
            ccounts[c] = total;
        } else {
            const int64_t e = orc_scan_find(ckeys, ccap, ORC_EMPTY_KEY);
            if (e >= 0) { ckeys[e] = dk[j]; ccounts[e] = total; }
        }
    }
    int64_t room = max_keys - stored;
    if (room < 0) room = 0;
    int64_t nvict = 0;
    if (mode != ORC_SCORE_NONE && ncand > room) {
        orc_victim* v = (orc_victim*)malloc(sizeof(orc_victim) * (size_t)(stored > 0 ? stored : 1));
        int64_t nv = 0;
        for (int64_t s = 0; s < capacity; ++s) {
            if (tkeys[s] == ORC_EMPTY_KEY || tkeys[s] == ORC_TOMBSTONE) continue;
            v[nv].score = tscores[s] < 0xfffffffeull ? tscores[s] : 0xfffffffeull;
            v[nv].key = tkeys[s];
            v[nv].slot = s;
            ++nv;
        }
        qsort(v, (size_t)nv, sizeof(orc_victim), orc_victim_cmp);
        nvict = ncand - room < nv ? ncand - room : nv;
        for (int64_t i = 0; i < nvict; ++i) {
            tkeys[v[i].slot] = ORC_TOMBSTONE;
            tscores[v[i].slot] = 0;
        }
        free(v);
    }
    int64_t admit = room + nvict < ncand ? room + nvict : ncand;
    for (int64_t q = 0; q < ncand; ++q) {
        const int64_t j = cand[q];
        const int64_t c = orc_scan_find(ckeys, ccap, dk[j]);
        if (q >= admit) {                       /* left out: the count is kept */
            if (c >= 0) ccounts[c] = ctot[q];
            else {
                const int64_t e = orc_scan_find(ckeys, ccap, ORC_EMPTY_KEY);
                if (e >= 0) { ckeys[e] = dk[j]; ccounts[e] = ctot[q]; }
            }
            continue;
        }
        if (c >= 0) ccounts[c] = 0;
        const uint64_t h = orc_mix64((uint64_t)dk[j]);
        int64_t at = orc_home(h, capacity), probes = 0;
        while (probes < capacity && tkeys[at] != ORC_EMPTY_KEY && tkeys[at] != ORC_TOMBSTONE) {
            at = (at + 1 == capacity) ? 0 : at + 1;
            ++probes;
        }
        if (probes == capacity) continue;       /* cannot happen: room was counted */
        tkeys[at] = dk[j];
        tdig[at] = orc_digest(h);
        memcpy(tvals + at * ORC_DIM, init_vals + df[j] * ORC_DIM, sizeof(float) * ORC_DIM);
        if (mode == ORC_SCORE_STEP) tscores[at] = step;
        if (mode == ORC_SCORE_LFU) tscores[at] = ctot[q];
    }
    for (int64_t i = 0; i < n; ++i)
        slot_out[i] = (keys[i] == ORC_EMPTY_KEY || keys[i] == ORC_TOMBSTONE)
                          ? -2 : orc_scan_find(tkeys, capacity, keys[i]);
    counts_out[0] = admit;
    counts_out[1] = nvict;
    counts_out[2] = ncand - admit;
    free(dk); free(df); free(dc); free(cand); free(ctot);
}
